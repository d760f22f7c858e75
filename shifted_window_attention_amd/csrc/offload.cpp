// Saved-state offload engine (include/swin_offload.h): asynchronous copies between device
// memory and pinned host memory on two copy streams, ordered after the caller's stream by
// events, with a ring of completion events addressed by tickets.
#include <hip/hip_runtime.h>

#include <new>
#include <string>
#include <vector>

#include "../../include/swin_offload.h"
#include "swin_internal.h"

struct swin_offload {
  int device = -1;
  int ring = 0;
  hipStream_t streams[2] = {nullptr, nullptr};  // 0: stores (D2H), 1: loads (H2D)
  std::vector<hipEvent_t> dep, done;            // per slot: the caller-stream point, the copy's end
  uint64_t next = 1;                            // next ticket
  uint64_t bytes[2] = {0, 0};
};

namespace {

swin_status fail(swin_status st, const std::string& msg) {
  swin::set_error(msg);
  return st;
}

swin_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SWIN_OK;
  swin::set_error(std::string(what) + ": " + hipGetErrorString(e));
  return SWIN_ERR_HIP;
}

swin_status check_current(const swin_offload* o) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != o->device)
    return fail(SWIN_ERR_ARG, "the engine's device is not the current device");
  return SWIN_OK;
}

// true if p is memory of the given kind (device memory of `device`, or pinned host memory)
bool pointer_is(const void* p, hipMemoryType want, int device) {
  hipPointerAttribute_t a{};
  const hipError_t e = hipPointerGetAttributes(&a, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // pageable host memory is reported as an invalid value
    return false;
  }
  if (a.type != want) return false;
  return want != hipMemoryTypeDevice || a.device == device;
}

swin_status issue(swin_offload* o, int dir, const void* src, void* dst, size_t bytes, void* after,
                  swin_ticket* ticket) {
  if (!o || !src || !dst || !ticket) return fail(SWIN_ERR_ARG, "NULL engine, pointer or ticket");
  *ticket = 0;
  if (bytes == 0) return fail(SWIN_ERR_ARG, "bytes must be > 0");
  swin_status st = check_current(o);
  if (st != SWIN_OK) return st;
  const void* dev = dir == 0 ? src : dst;
  const void* host = dir == 0 ? dst : src;
  if (!pointer_is(dev, hipMemoryTypeDevice, o->device))
    return fail(SWIN_ERR_ARG, "device pointer is not device memory of the engine's device");
  if (!pointer_is(host, hipMemoryTypeHost, o->device))
    return fail(SWIN_ERR_ARG, "host pointer is not pinned host memory");
  const uint64_t t = o->next;
  const int slot = (int)(t % (uint64_t)o->ring);
  hipError_t e = hipSuccess;
  if (t > (uint64_t)o->ring) e = hipEventSynchronize(o->done[slot]);  // the slot's previous copy
  if (e == hipSuccess) e = hipEventRecord(o->dep[slot], (hipStream_t)after);
  if (e == hipSuccess) e = hipStreamWaitEvent(o->streams[dir], o->dep[slot], 0);
  if (e == hipSuccess)
    e = hipMemcpyAsync(dst, src, bytes, dir == 0 ? hipMemcpyDeviceToHost : hipMemcpyHostToDevice, o->streams[dir]);
  if (e == hipSuccess) e = hipEventRecord(o->done[slot], o->streams[dir]);
  if (e != hipSuccess) return hip_status(e, dir == 0 ? "offload store" : "offload load");
  o->next = t + 1;
  o->bytes[dir] += bytes;
  *ticket = t;
  return SWIN_OK;
}

// slot of a live ticket, -1 for a ticket whose slot was reused (complete), or an error
swin_status ticket_slot(const swin_offload* o, swin_ticket t, int* slot) {
  if (!o) return fail(SWIN_ERR_ARG, "engine is NULL");
  if (t == 0 || t >= o->next) return fail(SWIN_ERR_ARG, "ticket was not issued by this engine");
  *slot = (t + (uint64_t)o->ring < o->next) ? -1 : (int)(t % (uint64_t)o->ring);
  return SWIN_OK;
}

void release(swin_offload* o) {
  for (hipEvent_t ev : o->dep)
    if (ev) (void)hipEventDestroy(ev);
  for (hipEvent_t ev : o->done)
    if (ev) (void)hipEventDestroy(ev);
  for (hipStream_t s : o->streams)
    if (s) (void)hipStreamDestroy(s);
  delete o;
}

}  // namespace

extern "C" {

swin_status swin_offload_create(int32_t ring, swin_offload** out) {
  if (!out) return fail(SWIN_ERR_ARG, "engine output is NULL");
  *out = nullptr;
  if (ring == 0) ring = 64;
  if (ring < 1 || ring > 4096) return fail(SWIN_ERR_ARG, "ring must be in [1, 4096] (0 = 64)");
  swin_offload* o = new (std::nothrow) swin_offload();
  if (!o) return fail(SWIN_ERR_ARG, "out of host memory");
  o->ring = ring;
  o->dep.assign(ring, nullptr);
  o->done.assign(ring, nullptr);
  hipError_t e = hipGetDevice(&o->device);
  for (int d = 0; d < 2 && e == hipSuccess; ++d) e = hipStreamCreateWithFlags(&o->streams[d], hipStreamNonBlocking);
  for (int i = 0; i < ring && e == hipSuccess; ++i) {
    e = hipEventCreateWithFlags(&o->dep[i], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&o->done[i], hipEventDisableTiming);
  }
  if (e != hipSuccess) {
    release(o);
    return hip_status(e, "offload engine creation");
  }
  *out = o;
  return SWIN_OK;
}

void swin_offload_destroy(swin_offload* engine) {
  if (!engine) return;
  for (hipStream_t s : engine->streams)
    if (s) (void)hipStreamSynchronize(s);
  release(engine);
}

swin_status swin_pinned_alloc(size_t bytes, void** host) {
  if (!host) return fail(SWIN_ERR_ARG, "host output is NULL");
  *host = nullptr;
  if (bytes == 0) return fail(SWIN_ERR_ARG, "bytes must be > 0");
  return hip_status(hipHostMalloc(host, bytes, hipHostMallocDefault), "pinned host allocation");
}

swin_status swin_pinned_free(void* host) {
  if (!host) return fail(SWIN_ERR_ARG, "host pointer is NULL");
  return hip_status(hipHostFree(host), "pinned host free");
}

swin_status swin_offload_store(swin_offload* engine, const void* dev, void* host, size_t bytes, void* after,
                               swin_ticket* ticket) {
  return issue(engine, 0, dev, host, bytes, after, ticket);
}

swin_status swin_offload_load(swin_offload* engine, const void* host, void* dev, size_t bytes, void* after,
                              swin_ticket* ticket) {
  return issue(engine, 1, host, dev, bytes, after, ticket);
}

swin_status swin_offload_wait(swin_offload* engine, swin_ticket ticket, void* stream) {
  int slot = 0;
  swin_status st = ticket_slot(engine, ticket, &slot);
  if (st != SWIN_OK || slot < 0) return st;
  st = check_current(engine);
  if (st != SWIN_OK) return st;
  return hip_status(hipStreamWaitEvent((hipStream_t)stream, engine->done[slot], 0), "offload wait");
}

swin_status swin_offload_query(swin_offload* engine, swin_ticket ticket, int32_t* done) {
  if (!done) return fail(SWIN_ERR_ARG, "done output is NULL");
  *done = 0;
  int slot = 0;
  swin_status st = ticket_slot(engine, ticket, &slot);
  if (st != SWIN_OK) return st;
  if (slot < 0) {
    *done = 1;
    return SWIN_OK;
  }
  const hipError_t e = hipEventQuery(engine->done[slot]);
  if (e == hipSuccess) {
    *done = 1;
    return SWIN_OK;
  }
  if (e == hipErrorNotReady) return SWIN_OK;
  return hip_status(e, "offload query");
}

swin_status swin_offload_sync(swin_offload* engine) {
  if (!engine) return fail(SWIN_ERR_ARG, "engine is NULL");
  hipError_t e = hipSuccess;
  for (int d = 0; d < 2 && e == hipSuccess; ++d) e = hipStreamSynchronize(engine->streams[d]);
  return hip_status(e, "offload sync");
}

swin_status swin_offload_bytes(const swin_offload* engine, uint64_t* stored, uint64_t* loaded) {
  if (!engine) return fail(SWIN_ERR_ARG, "engine is NULL");
  if (stored) *stored = engine->bytes[0];
  if (loaded) *loaded = engine->bytes[1];
  return SWIN_OK;
}

}  // extern "C"
