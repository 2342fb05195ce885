// Host side of pseudo-streaming (include/gigaam.h): the ring plan, the two copies a push
// needs, and the step as one gigaam_encode of the window.
//
// "GigaAM on MLX ...", section "Streaming: honestly, it's pseudo-streaming": a growing
// buffer, every step re-recognising all of the audio but no more than the last 30 s.
// Here the window is a parameter and the audio lives in a caller-owned device ring, so a
// step reads its window in place and no sample crosses PCIe twice.
#include <hip/hip_runtime.h>

#include "gigaam.h"
#include "host.h"
#include "kernels.h"

using namespace gg;

extern "C" int gigaam_stream_init(gigaam_stream_state* st, int32_t window, int32_t capacity) {
  if (!st) return fail(GIGAAM_E_INVAL, "NULL stream state");
  if (window < 320 || window > (1 << 29))
    return fail(GIGAAM_E_INVAL, "stream window %d outside [320, 2^29]", window);
  if (capacity < 2 * window)
    return fail(GIGAAM_E_INVAL, "ring capacity %d < 2 * window (%d)", capacity, 2 * window);
  st->total = 0;
  st->window = window;
  st->capacity = capacity;
  st->start = 0;
  st->length = 0;
  return GIGAAM_OK;
}

static int check_state(const gigaam_stream_state* st) {
  if (!st) return fail(GIGAAM_E_INVAL, "NULL stream state");
  if (st->window < 320 || st->capacity < 2 * st->window || st->start < 0 || st->length < 0 ||
      st->length > st->window || st->start + st->length > st->capacity || st->total < st->length)
    return fail(GIGAAM_E_INVAL, "stream state is not one gigaam_stream_init/push produced");
  return GIGAAM_OK;
}

extern "C" int gigaam_stream_plan_push(const gigaam_stream_state* st, int32_t n,
                                       gigaam_stream_plan* pl) {
  if (int rc = check_state(st)) return rc;
  if (!pl) return fail(GIGAAM_E_INVAL, "NULL plan");
  if (n < 0) return fail(GIGAAM_E_INVAL, "push of %d samples", n);
  const int32_t W = st->window;
  const int32_t m = n < W ? n : W;                    // chunk samples that can stay
  gigaam_stream_plan p{};
  p.append_len = m;
  p.skip = n - m;
  p.total = st->total + n;
  if ((int64_t)st->start + st->length + m <= st->capacity) {   // room after the window
    p.move_src = 0;
    p.move_len = 0;
    p.append_at = st->start + st->length;
    p.start = st->start;
    p.length = st->length + m;
    if (p.length > W) {
      p.start += p.length - W;
      p.length = W;
    }
  } else {                                            // move the retained tail to offset 0
    const int32_t keep = st->length < W - m ? st->length : W - m;
    p.move_src = st->start + st->length - keep;       // >= W >= keep + m: no overlap
    p.move_len = keep;
    p.append_at = keep;
    p.start = 0;
    p.length = keep + m;
  }
  *pl = p;
  return GIGAAM_OK;
}

extern "C" int gigaam_stream_push(gigaam_stream_state* st, float* ring, const float* pcm,
                                  int32_t n, void* hip_stream) {
  gigaam_stream_plan p;
  if (int rc = gigaam_stream_plan_push(st, n, &p)) return rc;
  if (!ring) return fail(GIGAAM_E_INVAL, "NULL ring");
  if (n > 0 && !pcm) return fail(GIGAAM_E_INVAL, "NULL pcm for a push of %d samples", n);
  hipStream_t s = (hipStream_t)hip_stream;
  if (p.move_len > 0) {
    const hipError_t e = launch_copy_f32(ring, ring + p.move_src, p.move_len, s);
    if (e != hipSuccess) return fail(GIGAAM_E_HIP, "ring move: %s", hipGetErrorString(e));
  }
  if (p.append_len > 0) {
    const hipError_t e = launch_copy_f32(ring + p.append_at, pcm + p.skip, p.append_len, s);
    if (e != hipSuccess) return fail(GIGAAM_E_HIP, "ring append: %s", hipGetErrorString(e));
  }
  st->total = p.total;
  st->start = p.start;
  st->length = p.length;
  return GIGAAM_OK;
}

extern "C" int gigaam_stream_step(gigaam_model* model, const gigaam_stream_state* st,
                                  const float* ring, void* workspace, size_t workspace_bytes,
                                  float* log_probs, int32_t* token_ids, int32_t* n_tokens,
                                  int32_t* frame_ids, float* enc_out, int32_t* n_frames,
                                  void* hip_stream) {
  if (int rc = check_state(st)) return rc;
  if (!ring) return fail(GIGAAM_E_INVAL, "NULL ring");
  if (st->length < 320)
    return fail(GIGAAM_E_INVAL, "%d samples buffered; a step needs at least 320", st->length);
  const int32_t len = st->length;
  return gigaam_encode(model, ring + st->start, &len, 1, len, workspace, workspace_bytes,
                       log_probs, token_ids, n_tokens, frame_ids, enc_out, n_frames, hip_stream);
}
