// liblinattn C-ABI front end: argument validation, work planning and kernel
// dispatch.  Every check runs on the host before anything is enqueued, so an
// argument error never leaves a half-written output.  No device memory is
// allocated here; the caller brings every buffer, including the workspace.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "liblinattn.h"
#include "la_launch.hpp"

#define LA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_msg[512] = "";

la_status fail(la_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return s;
}

la_status ok() {
  g_msg[0] = '\0';
  return LA_OK;
}

la_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(LA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// Workgroups that keep all 256 compute units of an MI355X busy with two
// resident chunk workgroups each.  A shape constant, not a device query, so
// that workspace sizes depend on the shape alone.
constexpr int64_t kTargetGroups = 512;
constexpr int64_t kChunk = 64;

bool head_size_ok(int64_t d) { return d == 32 || d == 64 || d == 128; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Range {
  uintptr_t lo, hi;
};
Range range(const void* p, int64_t bytes) {
  Range r;
  r.lo = (uintptr_t)p;
  r.hi = (uintptr_t)p + (uintptr_t)(bytes > 0 ? bytes : 0);
  return r;
}
bool overlap(Range a, Range b) {
  if (!a.lo || !b.lo || a.hi == a.lo || b.hi == b.lo) return false;
  return a.lo < b.hi && b.lo < a.hi;
}
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Split of a causal sequence into segments of chunks (shape-only).  `cap`
// bounds the workspace a split may use (bytes; SIZE_MAX = unbounded): with a
// smaller bound the sequence is cut into fewer, longer segments, down to one
// segment (no workspace).  `slot` is the bytes of one segment's state.
struct CausalPlan {
  int64_t nchunks, nseg, seg_chunks;
};
CausalPlan plan_causal(int64_t U, int64_t T, int64_t slot = 0, size_t cap = SIZE_MAX) {
  CausalPlan p;
  p.nchunks = ceil_div(T, kChunk);
  p.nseg = 1;
  p.seg_chunks = p.nchunks;
  if (U < kTargetGroups && p.nchunks > 1) {
    int64_t want = ceil_div(kTargetGroups, U);
    if (want > p.nchunks) want = p.nchunks;
    if (cap != SIZE_MAX) {
      const int64_t fit = (int64_t)(cap / (size_t)(U * slot));
      if (want > fit) want = fit;
    }
    if (want >= 2) {
      p.seg_chunks = ceil_div(p.nchunks, want);
      p.nseg = ceil_div(p.nchunks, p.seg_chunks);
    }
  }
  return p;
}

// Split of a non-causal reduction over T (shape-only), bounded like
// plan_causal; nsplit = 0 when not even one slot per unit fits `cap`.
struct NonCausalPlan {
  int64_t nchunks, nsplit, split_chunks;
};
NonCausalPlan plan_noncausal(int64_t U, int64_t T, int64_t slot = 0, size_t cap = SIZE_MAX) {
  NonCausalPlan p;
  p.nchunks = ceil_div(T, kChunk);
  int64_t want = ceil_div(kTargetGroups, U);
  if (want > p.nchunks) want = p.nchunks;
  if (want < 1) want = 1;
  if (cap != SIZE_MAX) {
    const int64_t fit = (int64_t)(cap / (size_t)(U * slot));
    if (want > fit) want = fit;
    if (want < 1) {
      p.nsplit = p.split_chunks = 0;
      return p;
    }
  }
  p.split_chunks = ceil_div(p.nchunks, want);
  p.nsplit = ceil_div(p.nchunks, p.split_chunks);
  return p;
}

int64_t state_elems(int64_t Dk, int64_t Dv, int norm) { return Dk * Dv + (norm ? Dk : 0); }

size_t forward_ws_bytes(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, int causal, int norm,
                        size_t cap = SIZE_MAX) {
  const int64_t U = B * H;
  if (U == 0 || T == 0) return 0;
  const int64_t slot = state_elems(Dk, Dv, norm) * 4;
  if (causal) {
    CausalPlan p = plan_causal(U, T, slot, cap);
    if (p.nseg <= 1) return 0;
    return (size_t)(U * p.nseg * slot);
  }
  NonCausalPlan p = plan_noncausal(U, T, slot, cap);
  return (size_t)(U * p.nsplit * slot);
}

static_assert(la::kIoF32 == LA_DT_F32 && la::kIoBF16 == LA_DT_BF16 && la::kIoF16 == LA_DT_F16,
              "launcher I/O codes are the la_dtype values");
bool dtype_ok(int32_t dtype) { return dtype == LA_DT_F32 || dtype == LA_DT_BF16 || dtype == LA_DT_F16; }
int64_t dtype_size(int32_t dtype) { return dtype == LA_DT_F32 ? 4 : 2; }

// unequal: Dk and Dv may differ (each 32, 64 or 128)
la_status check_common(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, int32_t dtype,
                       bool unequal = true) {
  if (!dtype_ok(dtype))
    return fail(LA_ERR_DTYPE, "dtype %d is not a supported floating type (0=f32, 1=bf16, 2=f16)", dtype);
  if (B < 0 || T < 0 || H < 1 || Dk < 1 || Dv < 1)
    return fail(LA_ERR_SHAPE, "bad sizes B=%lld T=%lld H=%lld Dk=%lld Dv=%lld", (long long)B,
                (long long)T, (long long)H, (long long)Dk, (long long)Dv);
  if (!head_size_ok(Dk) || !head_size_ok(Dv))
    return fail(LA_ERR_UNSUPPORTED, "head sizes Dk=%lld Dv=%lld: each must be 32, 64 or 128",
                (long long)Dk, (long long)Dv);
  if (!unequal && Dk != Dv)
    return fail(LA_ERR_UNSUPPORTED, "head sizes Dk=%lld Dv=%lld: this call needs Dk == Dv",
                (long long)Dk, (long long)Dv);
  if (B * H > (int64_t)1 << 30 || T > ((int64_t)1 << 31) - kChunk || H * Dk > (int64_t)1 << 30)
    return fail(LA_ERR_SHAPE, "sizes exceed the 32-bit index ranges of the kernels");
  return LA_OK;
}

}  // namespace

LA_EXPORT const char* la_status_string(la_status s) {
  switch (s) {
    case LA_OK: return "LA_OK";
    case LA_ERR_NULL_ARG: return "LA_ERR_NULL_ARG";
    case LA_ERR_DTYPE: return "LA_ERR_DTYPE";
    case LA_ERR_SHAPE: return "LA_ERR_SHAPE";
    case LA_ERR_STATE: return "LA_ERR_STATE";
    case LA_ERR_BAD_ARG: return "LA_ERR_BAD_ARG";
    case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED";
    case LA_ERR_WORKSPACE: return "LA_ERR_WORKSPACE";
    case LA_ERR_DEVICE: return "LA_ERR_DEVICE";
  }
  return "LA_ERR_UNKNOWN";
}

LA_EXPORT const char* la_last_error_message(void) { return g_msg; }

LA_EXPORT la_status la_initial_state(float* kv, float* k, int64_t B, int64_t H, int64_t Dk,
                                     int64_t Dv, void* stream) {
  if (B < 0 || H < 1 || Dk < 1 || Dv < 1) return fail(LA_ERR_SHAPE, "bad state sizes");
  if (!kv) return fail(LA_ERR_NULL_ARG, "kv state pointer is NULL");
  if (k && overlap(range(kv, B * H * Dk * Dv * 4), range(k, B * H * Dk * 4)))
    return fail(LA_ERR_BAD_ARG, "kv and k state buffers overlap");
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = la::launch_fill_zero(kv, B * H * Dk * Dv, st);
  if (e == hipSuccess && k) e = la::launch_fill_zero(k, B * H * Dk, st);
  return device_status(e, "la_initial_state");
}

LA_EXPORT la_status la_workspace_size(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                                      int32_t dtype, int32_t causal, size_t* bytes) {
  if (!bytes) return fail(LA_ERR_NULL_ARG, "bytes is NULL");
  la_status s = check_common(B, T, H, Dk, Dv, dtype);
  if (s != LA_OK) return s;
  // the normaliser adds Dk floats per slot; size for it so the answer does not
  // depend on use_normalizer
  *bytes = forward_ws_bytes(B, T, H, Dk, Dv, causal != 0, 1);
  return ok();
}

namespace {
// The allocation-free variant's scratch: one array per GPU the library runs
// on, held until the process ends.  Host code never uses the array's name as
// an address: scratch_for_stream() looks up each device's own copy once
// (hipGetSymbolAddress, with that device current) and keeps it.
constexpr size_t kScratchBytes = LA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

la_status scratch_for_stream(hipStream_t st, void** ptr) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return device_status(e, "la_forward_noalloc (hipGetDevice)");
  if (st) {
    hipDevice_t sd = 0;
    e = hipStreamGetDevice(st, &sd);
    if (e != hipSuccess) return device_status(e, "la_forward_noalloc (hipStreamGetDevice)");
    if ((int)sd != cur)
      return fail(LA_ERR_DEVICE, "la_forward_noalloc: the stream belongs to device %d, the current device is %d",
                  (int)sd, cur);
  }
  if (cur < 0 || cur >= kMaxDevices) return fail(LA_ERR_DEVICE, "device index %d out of range", cur);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[cur]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return device_status(e, "la_forward_noalloc (hipGetSymbolAddress)");
    if (!p) return fail(LA_ERR_DEVICE, "la_forward_noalloc: no address for the scratch array");
    g_scratch_ptr[cur] = p;
  }
  *ptr = g_scratch_ptr[cur];
  return LA_OK;
}

// la_forward; with noalloc the workspace is the device's scratch array and
// the split plans are bounded by its size.
la_status forward_impl(const void* q, const void* k, const void* v, const uint8_t* mask,
                       const float* state_in_kv, const float* state_in_k, float* state_out_kv,
                       float* state_out_k, int32_t causal, int32_t feature_map, int32_t use_normalizer,
                       float eps, void* out, int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                       int32_t dtype, void* workspace, size_t workspace_bytes, void* stream, bool noalloc) {
  const size_t cap = noalloc ? kScratchBytes : SIZE_MAX;
  la_status s = check_common(B, T, H, Dk, Dv, dtype);
  if (s != LA_OK) return s;
  if (feature_map != LA_FM_ELU_PLUS_ONE && feature_map != LA_FM_RELU_EPS)
    return fail(LA_ERR_BAD_ARG, "feature_map %d is not 0 (elu+1) or 1 (relu+eps)", feature_map);
  if (!(eps >= 0.f) || isinf(eps)) return fail(LA_ERR_BAD_ARG, "eps must be finite and >= 0");
  const int norm = use_normalizer != 0;
  const int64_t U = B * H;
  const int64_t esz = dtype_size(dtype);
  const bool work = U > 0 && T > 0;
  if (work && (!q || !k || !v || !out)) return fail(LA_ERR_NULL_ARG, "q, k, v and out are required");
  if (!causal) {
    if (state_in_kv || state_in_k || state_out_kv || state_out_k)
      return fail(LA_ERR_STATE, "non-causal attention does not take or return a state");
  } else if (!norm) {
    if (state_in_k || state_out_k)
      return fail(LA_ERR_STATE, "use_normalizer=0 carries only the kv state; k parts must be NULL");
  } else {
    if ((state_in_kv != nullptr) != (state_in_k != nullptr))
      return fail(LA_ERR_STATE, "normalized state_in needs both kv and k (or neither)");
    if ((state_out_kv != nullptr) != (state_out_k != nullptr))
      return fail(LA_ERR_STATE, "normalized state_out needs both kv and k (or neither)");
  }
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      !aligned16(state_in_kv) || !aligned16(state_out_kv))
    return fail(LA_ERR_BAD_ARG, "q, k, v, out and kv states must be 16-byte aligned");
  if (!aligned16(state_in_k) || !aligned16(state_out_k) || !aligned16(workspace))
    return fail(LA_ERR_BAD_ARG, "k states and workspace must be 16-byte aligned");

  const int64_t nqk = B * T * H * Dk * esz, nvo = B * T * H * Dv * esz;
  const Range rq = range(q, nqk), rk = range(k, nqk), rv = range(v, nvo), ro = range(out, nvo);
  const Range rm = range(mask, B * T);
  const Range rsi = range(state_in_kv, U * Dk * Dv * 4), rzi = range(state_in_k, U * Dk * 4);
  const Range rso = range(state_out_kv, U * Dk * Dv * 4), rzo = range(state_out_k, U * Dk * 4);
  const size_t need = forward_ws_bytes(B, T, H, Dk, Dv, causal != 0, norm, cap);
  const int64_t slot = state_elems(Dk, Dv, norm) * 4;
  if (noalloc && work && !causal && plan_noncausal(U, T, slot, cap).nsplit == 0)
    return fail(LA_ERR_WORKSPACE,
                "la_forward_noalloc: the non-causal sums of %lld (batch, head) units need %lld bytes, "
                "more than the %zu-byte scratch",
                (long long)U, (long long)(U * slot), kScratchBytes);
  if (noalloc) workspace = nullptr;  // the scratch array, looked up below
  const Range rw = range(workspace, (int64_t)need);
  if (overlap(ro, rq) || overlap(ro, rk) || overlap(ro, rv) || overlap(ro, rm) || overlap(ro, rsi) ||
      overlap(ro, rzi) || overlap(ro, rso) || overlap(ro, rzo))
    return fail(LA_ERR_BAD_ARG, "out overlaps another argument");
  if (overlap(rso, rzo) || overlap(rsi, rzi))
    return fail(LA_ERR_BAD_ARG, "kv and k state buffers overlap");
  const Range outs[2] = {rso, rzo};
  const Range ins[5] = {rq, rk, rv, rm, rw};
  for (const Range& o : outs)
    for (const Range& i : ins)
      if (overlap(o, i)) return fail(LA_ERR_BAD_ARG, "state_out overlaps an input or the workspace");
  if ((overlap(rso, rsi) && state_out_kv != state_in_kv) ||
      (overlap(rzo, rzi) && state_out_k != state_in_k) || overlap(rso, rzi) || overlap(rzo, rsi))
    return fail(LA_ERR_BAD_ARG, "state_out may equal state_in exactly but not partially overlap it");
  if (overlap(rw, rq) || overlap(rw, rk) || overlap(rw, rv) || overlap(rw, rm) || overlap(rw, rsi) ||
      overlap(rw, rzi))
    return fail(LA_ERR_BAD_ARG, "workspace overlaps an input");
  if (!noalloc && need > 0 && (!workspace || workspace_bytes < need))
    return fail(LA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);

  hipStream_t st = (hipStream_t)stream;
  if (noalloc && need > 0) {
    s = scratch_for_stream(st, &workspace);
    if (s != LA_OK) return s;
  }
  // the kernels' tile size: the larger head size (the smaller side zero-padded)
  const int Di = (int)(Dk > Dv ? Dk : Dv);
  hipError_t e = hipSuccess;

  if (!work) {
    // nothing to read: a causal state passes through unchanged (zeros if none)
    if (causal && state_out_kv) {
      const int64_t n = U * Dk * Dv;
      e = (state_in_kv) ? (state_out_kv != state_in_kv ? la::launch_copy(state_out_kv, state_in_kv, n, st)
                                                       : hipSuccess)
                        : la::launch_fill_zero(state_out_kv, n, st);
      if (e == hipSuccess && norm)
        e = state_in_k ? (state_out_k != state_in_k ? la::launch_copy(state_out_k, state_in_k, U * Dk, st)
                                                    : hipSuccess)
                       : la::launch_fill_zero(state_out_k, U * Dk, st);
    }
    return device_status(e, "la_forward");
  }

  la::ChunkArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.mask = mask;
  a.out = out;
  a.T = (int32_t)T;
  a.H = (int32_t)H;
  a.eps = eps;
  a.dk = Dk != Dv ? (int32_t)Dk : 0;
  a.dv = Dk != Dv ? (int32_t)Dv : 0;
  const int64_t SE = Dk * Dv, ZE = Dk;

  if (causal) {
    CausalPlan p = plan_causal(U, T, slot, cap);
    if (p.nseg == 1) {
      a.s_in = state_in_kv;
      a.z_in = state_in_k;
      a.s_in_u = SE;
      a.z_in_u = ZE;
      a.s_out = state_out_kv;
      a.z_out = state_out_k;
      a.s_out_u = SE;
      a.z_out_u = ZE;
      a.seg_count = 1;
      a.seg_first = 0;
      a.seg_chunks = (int32_t)p.nchunks;
      a.nseg_total = 1;
      e = la::launch_chunk(la::kModeCausal, dtype, Di, feature_map, norm, a, (int)U, st);
      return device_status(e, "la_forward (causal)");
    }
    // split sequence: partial states of segments 0..nseg-2 -> slots 1..nseg-1,
    // exclusive prefix (slot 0 = state_in), then every segment from its prefix.
    float* ws_s = (float*)workspace;
    float* ws_z = norm ? ws_s + U * p.nseg * SE : nullptr;
    la::ChunkArgs ps = a;
    ps.s_out = ws_s;
    ps.z_out = ws_z;
    ps.s_out_u = p.nseg * SE;
    ps.s_out_s = SE;
    ps.z_out_u = p.nseg * ZE;
    ps.z_out_s = ZE;
    ps.out_slot_off = 1;
    ps.seg_count = (int32_t)(p.nseg - 1);
    ps.seg_first = 0;
    ps.seg_chunks = (int32_t)p.seg_chunks;
    ps.nseg_total = (int32_t)p.nseg;
    e = la::launch_chunk(la::kModeState, dtype, Di, feature_map, norm, ps, (int)(U * (p.nseg - 1)), st);
    // up to kChunkFold segments the causal pass adds the slots itself, reading
    // the initial state in every segment; a state updated in place goes
    // through the prefix pass instead (its slot 0 holds the initial state), so
    // that no segment reads it after the last one has written it
    const bool in_place = (state_in_kv && state_in_kv == state_out_kv) || (state_in_k && state_in_k == state_out_k);
    const bool fold = p.nseg <= la::kChunkFold && Di <= 64 && !in_place;
    if (e == hipSuccess && !fold)
      e = la::launch_seg_prefix(ws_s, ws_z, state_in_kv, state_in_k, (int)U, (int)p.nseg, (int)Dk, (int)Dv, norm,
                                st);
    if (e == hipSuccess) {
      la::ChunkArgs pc = a;
      pc.fold = fold ? 1 : 0;
      pc.s_init = state_in_kv;
      pc.z_init = state_in_k;
      pc.s_init_u = SE;
      pc.z_init_u = ZE;
      pc.s_in = ws_s;
      pc.z_in = ws_z;
      pc.s_in_u = p.nseg * SE;
      pc.s_in_s = SE;
      pc.z_in_u = p.nseg * ZE;
      pc.z_in_s = ZE;
      pc.s_out = state_out_kv;
      pc.z_out = state_out_k;
      pc.s_out_u = SE;
      pc.z_out_u = ZE;
      pc.seg_count = (int32_t)p.nseg;
      pc.seg_first = 0;
      pc.seg_chunks = (int32_t)p.seg_chunks;
      pc.nseg_total = (int32_t)p.nseg;
      e = la::launch_chunk(la::kModeCausal, dtype, Di, feature_map, norm, pc, (int)(U * p.nseg), st);
    }
    return device_status(e, "la_forward (causal, split)");
  }

  // non-causal: split reduction -> fixed-order sum -> readout
  NonCausalPlan p = plan_noncausal(U, T, slot, cap);
  float* ws_s = (float*)workspace;
  float* ws_z = norm ? ws_s + U * p.nsplit * SE : nullptr;
  la::ChunkArgs pr = a;
  pr.s_out = ws_s;
  pr.z_out = ws_z;
  pr.s_out_u = p.nsplit * SE;
  pr.s_out_s = SE;
  pr.z_out_u = p.nsplit * ZE;
  pr.z_out_s = ZE;
  pr.out_slot_off = 0;
  pr.seg_count = (int32_t)p.nsplit;
  pr.seg_first = 0;
  pr.seg_chunks = (int32_t)p.split_chunks;
  pr.nseg_total = (int32_t)p.nsplit;
  pr.chunk_step = (int32_t)p.nsplit;  // split s sums chunks s, s + nsplit, ...: masked tails spread
  e = la::launch_chunk(la::kModeState, dtype, Di, feature_map, norm, pr, (int)(U * p.nsplit), st);
  if (e == hipSuccess) e = la::launch_seg_sum(ws_s, ws_z, (int)U, (int)p.nsplit, (int)Dk, (int)Dv, norm, st);
  if (e == hipSuccess) {
    la::ApplyArgs pa;
    pa.q = a.q;
    pa.mask = a.mask;
    pa.out = a.out;
    pa.s = ws_s;
    pa.z = ws_z;
    pa.s_u = p.nsplit * SE;
    pa.z_u = p.nsplit * ZE;
    pa.T = a.T;
    pa.H = a.H;
    pa.seg_count = la::apply_groups_per_unit(U, T);
    pa.eps = a.eps;
    pa.dk = a.dk;
    pa.dv = a.dv;
    e = la::launch_apply(dtype, Di, feature_map, norm, pa, (int)(U * pa.seg_count), st);
  }
  return device_status(e, "la_forward (non-causal)");
}
}  // namespace

LA_EXPORT la_status la_forward(const void* q, const void* k, const void* v, const uint8_t* mask,
                               const float* state_in_kv, const float* state_in_k,
                               float* state_out_kv, float* state_out_k, int32_t causal,
                               int32_t feature_map, int32_t use_normalizer, float eps, void* out,
                               int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                               int32_t dtype, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return forward_impl(q, k, v, mask, state_in_kv, state_in_k, state_out_kv, state_out_k, causal, feature_map,
                      use_normalizer, eps, out, B, T, H, Dk, Dv, dtype, workspace, workspace_bytes, stream, false);
}

LA_EXPORT la_status la_forward_noalloc(const void* q, const void* k, const void* v, const uint8_t* mask,
                                       const float* state_in_kv, const float* state_in_k,
                                       float* state_out_kv, float* state_out_k, int32_t causal,
                                       int32_t feature_map, int32_t use_normalizer, float eps, void* out,
                                       int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                                       int32_t dtype, void* stream) {
  return forward_impl(q, k, v, mask, state_in_kv, state_in_k, state_out_kv, state_out_k, causal, feature_map,
                      use_normalizer, eps, out, B, T, H, Dk, Dv, dtype, nullptr, 0, stream, true);
}

LA_EXPORT la_status la_step(const void* q, const void* k, const void* v, const uint8_t* mask,
                            const float* state_in_kv, const float* state_in_k,
                            float* state_out_kv, float* state_out_k, int32_t feature_map,
                            int32_t use_normalizer, float eps, void* out, int64_t B, int64_t H,
                            int64_t Dk, int64_t Dv, int32_t dtype, void* stream) {
  la_status s = check_common(B, 1, H, Dk, Dv, dtype);
  if (s != LA_OK) return s;
  if (feature_map != LA_FM_ELU_PLUS_ONE && feature_map != LA_FM_RELU_EPS)
    return fail(LA_ERR_BAD_ARG, "feature_map %d is not 0 (elu+1) or 1 (relu+eps)", feature_map);
  if (!(eps >= 0.f) || isinf(eps)) return fail(LA_ERR_BAD_ARG, "eps must be finite and >= 0");
  const int norm = use_normalizer != 0;
  const int64_t U = B * H;
  const int64_t esz = dtype_size(dtype);
  if (U == 0) return ok();
  if (!q || !k || !v || !out) return fail(LA_ERR_NULL_ARG, "q, k, v and out are required");
  if (!state_in_kv || !state_out_kv)
    return fail(LA_ERR_STATE, "a decode step needs state_in and state_out (kv)");
  if (norm && (!state_in_k || !state_out_k))
    return fail(LA_ERR_STATE, "use_normalizer=1 needs the k state in and out");
  if (!norm && (state_in_k || state_out_k))
    return fail(LA_ERR_STATE, "use_normalizer=0 carries only the kv state; k parts must be NULL");
  if (!aligned16(state_in_kv) || !aligned16(state_out_kv))
    return fail(LA_ERR_BAD_ARG, "kv states must be 16-byte aligned");
  const Range rq = range(q, U * Dk * esz), rk = range(k, U * Dk * esz), rv = range(v, U * Dv * esz);
  const Range ro = range(out, U * Dv * esz), rm = range(mask, B);
  const Range rsi = range(state_in_kv, U * Dk * Dv * 4), rzi = range(state_in_k, U * Dk * 4);
  const Range rso = range(state_out_kv, U * Dk * Dv * 4), rzo = range(state_out_k, U * Dk * 4);
  const Range ins[4] = {rq, rk, rv, rm};
  const Range outs[3] = {ro, rso, rzo};
  for (const Range& o : outs)
    for (const Range& i : ins)
      if (overlap(o, i)) return fail(LA_ERR_BAD_ARG, "an output overlaps q, k, v or mask");
  if (overlap(ro, rsi) || overlap(ro, rzi) || overlap(ro, rso) || overlap(ro, rzo))
    return fail(LA_ERR_BAD_ARG, "out overlaps a state buffer");
  if ((overlap(rso, rsi) && state_out_kv != state_in_kv) ||
      (overlap(rzo, rzi) && state_out_k != state_in_k) || overlap(rso, rzo) || overlap(rsi, rzi) ||
      overlap(rso, rzi) || overlap(rzo, rsi))
    return fail(LA_ERR_BAD_ARG, "state_out may equal state_in exactly but not partially overlap it");
  la::DecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.mask = mask;
  a.s_in = state_in_kv;
  a.z_in = state_in_k;
  a.s_out = state_out_kv;
  a.z_out = state_out_k;
  a.out = out;
  a.H = (int32_t)H;
  a.units = (int32_t)U;
  a.eps = eps;
  hipError_t e = la::launch_decode(dtype, (int)Dk, (int)Dv, feature_map, norm, a, (int)U,
                                   (hipStream_t)stream);
  return device_status(e, "la_step");
}

// ---------------------------------------------------------------------------
// gated GQA recurrence

namespace {
struct GatedPlan {
  int64_t nchunks, nseg, seg_chunks;
};
GatedPlan plan_gated(int64_t U, int64_t T) {
  GatedPlan p;
  p.nchunks = ceil_div(T, kChunk);
  p.nseg = 1;
  p.seg_chunks = p.nchunks;
  if (U < kTargetGroups && p.nchunks > 1) {
    int64_t want = ceil_div(kTargetGroups, U);
    if (want > p.nchunks) want = p.nchunks;
    p.seg_chunks = ceil_div(p.nchunks, want);
    p.nseg = ceil_div(p.nchunks, p.seg_chunks);
  }
  return p;
}
// bytes of the split's state slots and decay factors (0 without a split)
size_t gated_split_bytes(int64_t U, const GatedPlan& p, int64_t D, bool per_dim) {
  if (p.nseg <= 1) return 0;
  // slots of D*D floats plus the decay factors of each slot (one, or one per
  // key dim), padded to 16 bytes
  const int64_t na = U * p.nseg * (per_dim ? D : 1);
  return (size_t)(U * p.nseg * D * D * 4 + ceil_div(na, 4) * 16);
}
size_t gated_ws_bytes(int64_t B, int64_t T, int64_t Hkv, int64_t D, bool per_dim) {
  const int64_t U = B * Hkv;
  if (U == 0 || T <= 1) return 0;
  GatedPlan p = plan_gated(U, T);
  // a per-dim decay adds one strong-decay flag per (unit, segment)
  return gated_split_bytes(U, p, D, per_dim) + (per_dim ? (size_t)ceil_div(U * p.nseg, 4) * 16 : 0);
}
la_status check_gated(int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t Dk, int64_t Dv,
                      int32_t dtype) {
  if (!dtype_ok(dtype))
    return fail(LA_ERR_DTYPE, "dtype %d is not a supported floating type (0=f32, 1=bf16, 2=f16)", dtype);
  if (B < 0 || T < 0 || Hq < 1 || Hkv < 1 || Dk < 1 || Dv < 1)
    return fail(LA_ERR_SHAPE, "bad sizes");
  if (Hq % Hkv != 0)
    return fail(LA_ERR_SHAPE, "q_num_heads (%lld) must be a positive multiple of kv_num_heads (%lld)",
                (long long)Hq, (long long)Hkv);
  if (Dk != Dv || !head_size_ok(Dk))
    return fail(LA_ERR_UNSUPPORTED, "head sizes Dk=%lld Dv=%lld: only Dk == Dv in {32,64,128}",
                (long long)Dk, (long long)Dv);
  if (B * Hq > (int64_t)1 << 30 || T > ((int64_t)1 << 31) - kChunk || Hq * Dk > (int64_t)1 << 30)
    return fail(LA_ERR_SHAPE, "sizes exceed the 32-bit index ranges of the kernels");
  return LA_OK;
}
}  // namespace

// The chunk kernels take 1, 2, 4 or 8 query heads per workgroup: a kv head
// with G query heads runs as G / head_tile(G) workgroups (query-head groups)
// of head_tile(G) heads each, every one of them computing the kv head's
// recurrence and the first writing the state.
int64_t head_tile(int64_t G) { return G % 8 == 0 ? 8 : (G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1)); }

hipError_t launch_step(const void* q, const void* k, const void* v, const void* decay, bool per_dim,
                       const float* past_state, float* present_state, void* out, int64_t U,
                       int64_t Hkv, int64_t D, int64_t G, int32_t dtype, float scale, hipStream_t st) {
  la::GatedStepArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.decay = decay;
  a.per_dim = per_dim ? 1 : 0;
  a.s_in = past_state;
  a.s_out = present_state;
  a.out = out;
  a.Hkv = (int32_t)Hkv;
  a.units = (int32_t)U;
  a.scale = scale;
  return la::launch_gated_step(dtype, (int)D, (int)G, a, st);
}

namespace {
// fp32 inputs at head size 128 with a per-key-dim decay: the chunk kernels'
// fp32 tiles and decay table exceed the LDS, so T > 1 runs the whole-sequence
// token-by-token kernel (la_recur.hip: one launch, the state in registers; no
// workspace)
bool by_token(bool per_dim, int32_t dtype, int64_t D, int64_t T) {
  return per_dim && dtype == LA_DT_F32 && D == 128 && T > 1;
}

hipError_t launch_by_token(const void* q, const void* k, const void* v, const void* decay, const void* beta,
                           int64_t beta_heads, int delta, const float* past_state, float* present_state,
                           void* out, int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t D, int32_t dtype,
                           float scale, hipStream_t st) {
  const int64_t G = Hq / Hkv, GW = head_tile(G);
  la::RecurArgs r;
  memset(&r, 0, sizeof(r));
  r.q = q;
  r.k = k;
  r.v = v;
  r.decay = decay;
  r.beta = beta;
  r.out = out;
  r.s_in = past_state;
  r.s_out = present_state;
  r.T = (int32_t)T;
  r.Hq = (int32_t)Hq;
  r.Hkv = (int32_t)Hkv;
  r.units = (int32_t)(B * Hkv);
  r.beta_heads = (int32_t)beta_heads;
  r.hsplit = (int32_t)(G / GW);
  r.scale = scale;
  return la::launch_recur(dtype, (int)D, (int)GW, 2, delta, r, st);
}
}  // namespace

LA_EXPORT la_status la_gated_workspace_size(int64_t B, int64_t T, int64_t Hq, int64_t Hkv,
                                            int64_t Dk, int64_t Dv, int32_t dtype,
                                            int32_t per_dim_decay, size_t* bytes) {
  if (!bytes) return fail(LA_ERR_NULL_ARG, "bytes is NULL");
  la_status s = check_gated(B, T, Hq, Hkv, Dk, Dv, dtype);
  if (s != LA_OK) return s;
  *bytes = by_token(per_dim_decay != 0, dtype, Dk, T) ? 0 : gated_ws_bytes(B, T, Hkv, Dk, per_dim_decay != 0);
  return ok();
}

namespace {
// la_gated_forward, optionally in reversed time (reverse = 1: token t of the
// recurrence is row T-1-t of q, k, v and out; the backward pass's reverse sums
// run this way on its time-ordered buffers; not with a per-dim decay).
la_status gated_forward(const void* q, const void* k, const void* v, const void* decay,
                        int32_t per_dim_decay, const float* past_state, float* present_state, void* out,
                        int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t Dk, int64_t Dv,
                        int32_t dtype, float scale, void* workspace, size_t workspace_bytes, void* stream,
                        int32_t reverse) {
  la_status s = check_gated(B, T, Hq, Hkv, Dk, Dv, dtype);
  if (s != LA_OK) return s;
  if (isnan(scale) || isinf(scale)) return fail(LA_ERR_BAD_ARG, "scale must be finite");
  const int64_t D = Dk, U = B * Hkv, G = Hq / Hkv;
  const int64_t esz = dtype_size(dtype);
  const bool per_dim = per_dim_decay != 0 && decay != nullptr;
  if (reverse && per_dim) return fail(LA_ERR_UNSUPPORTED, "reversed time with a per-dim decay");
  if (per_dim && !aligned16(decay)) return fail(LA_ERR_BAD_ARG, "a per-dim decay must be 16-byte aligned");
  if (U > 0 && !present_state) return fail(LA_ERR_NULL_ARG, "present_state is required");
  const bool work = U > 0 && T > 0;
  if (work && (!q || !k || !v || !out)) return fail(LA_ERR_NULL_ARG, "q, k, v and out are required");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(past_state) ||
      !aligned16(present_state) || !aligned16(workspace))
    return fail(LA_ERR_BAD_ARG, "tensors and workspace must be 16-byte aligned");
  const Range rq = range(q, B * T * Hq * D * esz), rk = range(k, B * T * Hkv * D * esz);
  const Range rv = range(v, B * T * Hkv * D * esz), ro = range(out, B * T * Hq * D * esz);
  const Range rg = range(decay, B * T * Hkv * (per_dim ? D : 1) * esz);
  const Range rpi = range(past_state, U * D * D * 4), rpo = range(present_state, U * D * D * 4);
  const bool tokens = by_token(per_dim, dtype, D, T);
  const size_t need = tokens ? 0 : gated_ws_bytes(B, T, Hkv, D, per_dim);
  const Range rw = range(workspace, (int64_t)need);
  const Range ins[5] = {rq, rk, rv, rg, rw};
  for (const Range& i : ins)
    if (overlap(ro, i) || overlap(rpo, i)) return fail(LA_ERR_BAD_ARG, "an output overlaps an input");
  if (overlap(ro, rpi) || overlap(ro, rpo) || overlap(rw, rpi) || overlap(rw, rq) || overlap(rw, rk) ||
      overlap(rw, rv) || overlap(rw, rg))
    return fail(LA_ERR_BAD_ARG, "buffers overlap");
  if (overlap(rpo, rpi) && present_state != past_state)
    return fail(LA_ERR_BAD_ARG, "present_state may equal past_state exactly but not partially overlap it");
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(LA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (scale == 0.f) scale = 1.f / sqrtf((float)D);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (!work) {
    if (U > 0)
      e = past_state ? (present_state != past_state
                            ? la::launch_copy(present_state, past_state, U * D * D, st)
                            : hipSuccess)
                     : la::launch_fill_zero(present_state, U * D * D, st);
    return device_status(e, "la_gated_forward");
  }
  if (T == 1) {
    // one token: the state-streaming step kernel (no chunk to tile)
    e = launch_step(q, k, v, decay, per_dim, past_state, present_state, out, U, Hkv, D, G, dtype,
                    scale, st);
    return device_status(e, "la_gated_forward");
  }
  if (tokens) {
    e = launch_by_token(q, k, v, decay, nullptr, 0, 0, past_state, present_state, out, B, T, Hq, Hkv, D, dtype,
                        scale, st);
    return device_status(e, "la_gated_forward (token by token)");
  }
  const int64_t GW = head_tile(G), HS = G / GW;  // heads per workgroup, query-head groups
  // the output passes run HS workgroups per (unit, segment), query-head groups
  // first .. first + count - 1 per launch; the state pass one
  auto launch_groups = [&](int mode, const la::GatedArgs& ga, int grid, int64_t first, int64_t count) {
    la::GatedArgs g2 = ga;
    const bool grouped = mode != la::kModeState;
    g2.hsplit = grouped ? (int32_t)HS : 1;
    g2.hg_first = grouped ? (int32_t)first : 0;
    g2.hg_count = grouped ? (int32_t)count : 1;
    const int gr = (int)(grid * g2.hg_count);
    return per_dim ? la::launch_gated_pd(mode, dtype, (int)D, (int)GW, g2, gr, st)
                   : la::launch_gated(mode, dtype, (int)D, (int)GW, g2, gr, st);
  };
  // the output pass over grid (unit, segment) workgroups per query-head group;
  // with a per-dim decay, then the re-evaluation of its flagged segments.  A
  // state updated in place by several groups that each read it at their start:
  // the groups that only read it run first, then group 0, which also writes it.
  auto launch_out = [&](const la::GatedArgs& ga, int grid, bool in_place) {
    hipError_t r = hipSuccess;
    for (int pass = 0; pass < (per_dim ? 2 : 1) && r == hipSuccess; ++pass) {
      const int mode = pass == 0 ? la::kModeCausal : la::kModeRerun;
      if (in_place && HS > 1) {
        r = launch_groups(mode, ga, grid, 1, HS - 1);
        if (r == hipSuccess) r = launch_groups(mode, ga, grid, 0, 1);
      } else {
        r = launch_groups(mode, ga, grid, 0, HS);
      }
    }
    return r;
  };
  la::GatedArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.decay = decay;
  a.out = out;
  a.T = (int32_t)T;
  a.Hq = (int32_t)Hq;
  a.Hkv = (int32_t)Hkv;
  a.scale = scale;
  a.reverse = reverse;
  const int64_t SE = D * D;
  GatedPlan p = plan_gated(U, T);
  if (per_dim) a.flags = (int32_t*)((char*)workspace + gated_split_bytes(U, p, D, true));
  if (p.nseg == 1) {
    a.s_in = past_state;
    a.s_in_u = SE;
    a.s_out = present_state;
    a.s_out_u = SE;
    a.seg_count = 1;
    a.seg_chunks = (int32_t)p.nchunks;
    a.nseg_total = 1;
    e = launch_out(a, (int)U, past_state && past_state == present_state);
    return device_status(e, "la_gated_forward");
  }
  float* ws_s = (float*)workspace;
  float* ws_a = ws_s + U * p.nseg * SE;
  la::GatedArgs ps = a;
  ps.s_out = ws_s;
  ps.s_out_u = p.nseg * SE;
  ps.s_out_s = SE;
  ps.a_out = ws_a;
  ps.out_slot_off = 1;
  ps.seg_count = (int32_t)(p.nseg - 1);
  ps.seg_chunks = (int32_t)p.seg_chunks;
  ps.nseg_total = (int32_t)p.nseg;
  e = launch_groups(la::kModeState, ps, (int)(U * (p.nseg - 1)), 0, 1);
  if (e == hipSuccess)
    e = la::launch_gated_prefix(ws_s, ws_a, past_state, (int)U, (int)p.nseg, (int)D, per_dim ? 1 : 0, st);
  if (e == hipSuccess) {
    la::GatedArgs pc = a;
    pc.s_in = ws_s;
    pc.s_in_u = p.nseg * SE;
    pc.s_in_s = SE;
    pc.s_out = present_state;
    pc.s_out_u = SE;
    pc.seg_count = (int32_t)p.nseg;
    pc.seg_chunks = (int32_t)p.seg_chunks;
    pc.nseg_total = (int32_t)p.nseg;
    e = launch_out(pc, (int)(U * p.nseg), false);
  }
  return device_status(e, "la_gated_forward (split)");
}
}  // namespace

LA_EXPORT la_status la_gated_forward(const void* q, const void* k, const void* v,
                                     const void* decay, int32_t per_dim_decay,
                                     const float* past_state, float* present_state, void* out,
                                     int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t Dk,
                                     int64_t Dv, int32_t dtype, float scale, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return gated_forward(q, k, v, decay, per_dim_decay, past_state, present_state, out, B, T, Hq, Hkv, Dk, Dv,
                       dtype, scale, workspace, workspace_bytes, stream, 0);
}

LA_EXPORT la_status la_gated_step(const void* q, const void* k, const void* v, const void* decay,
                                  int32_t per_dim_decay, const float* past_state,
                                  float* present_state, void* out, int64_t B, int64_t Hq,
                                  int64_t Hkv, int64_t Dk, int64_t Dv, int32_t dtype, float scale,
                                  void* stream) {
  la_status s = check_gated(B, 1, Hq, Hkv, Dk, Dv, dtype);
  if (s != LA_OK) return s;
  if (isnan(scale) || isinf(scale)) return fail(LA_ERR_BAD_ARG, "scale must be finite");
  const int64_t D = Dk, U = B * Hkv, G = Hq / Hkv;
  const int64_t esz = dtype_size(dtype);
  if (U == 0) return ok();
  if (!q || !k || !v || !out || !present_state)
    return fail(LA_ERR_NULL_ARG, "q, k, v, out and present_state are required");
  if (!aligned16(past_state) || !aligned16(present_state))
    return fail(LA_ERR_BAD_ARG, "states must be 16-byte aligned");
  const Range rq = range(q, B * Hq * D * esz), rk = range(k, U * D * esz), rv = range(v, U * D * esz);
  const bool per_dim = per_dim_decay != 0 && decay != nullptr;
  const Range ro = range(out, B * Hq * D * esz), rg = range(decay, U * (per_dim ? D : 1) * esz);
  const Range rpi = range(past_state, U * D * D * 4), rpo = range(present_state, U * D * D * 4);
  const Range ins[4] = {rq, rk, rv, rg};
  for (const Range& i : ins)
    if (overlap(ro, i) || overlap(rpo, i)) return fail(LA_ERR_BAD_ARG, "an output overlaps an input");
  if (overlap(ro, rpi) || overlap(ro, rpo)) return fail(LA_ERR_BAD_ARG, "out overlaps a state buffer");
  if (overlap(rpo, rpi) && present_state != past_state)
    return fail(LA_ERR_BAD_ARG, "present_state may equal past_state exactly but not partially overlap it");
  if (scale == 0.f) scale = 1.f / sqrtf((float)D);
  hipError_t e = launch_step(q, k, v, decay, per_dim, past_state, present_state, out, U, Hkv, D, G,
                             dtype, scale, (hipStream_t)stream);
  return device_status(e, "la_gated_step");
}

// ---------------------------------------------------------------------------
// delta rules

namespace {
// Split of a delta-rule sequence over T (shape-only): with at most 64 (unit,
// query-head group) workgroups, segments of whole chunks (at least 4 each)
// bring the count towards 256; nseg = 1: no split.
struct DeltaPlan {
  int64_t nseg, seg_len;
};
DeltaPlan plan_delta(int64_t U, int64_t hs, int64_t T) {
  DeltaPlan p{1, T};
  const int64_t groups = U * hs, nchunks = ceil_div(T, kChunk);
  if (groups <= 0 || groups > 64) return p;
  int64_t want = ceil_div(256, groups);
  if (want > nchunks / 4) want = nchunks / 4;
  if (want < 2) return p;
  const int64_t seg_chunks = ceil_div(nchunks, want);
  p.nseg = ceil_div(nchunks, seg_chunks);
  p.seg_len = seg_chunks * kChunk;
  return p;
}
// workspace of a split: the maps M and N of every segment but the last, the
// start state of every segment, and the identity
size_t delta_ws_bytes(int64_t U, int64_t D, const DeltaPlan& p) {
  if (p.nseg <= 1) return 0;
  return (size_t)D * D * 4 * (size_t)(U * (p.nseg - 1) * 2 + U * p.nseg + 1);
}
}  // namespace

LA_EXPORT la_status la_delta_workspace_size(int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t Dk, int64_t Dv,
                                            int32_t dtype, int32_t per_dim_decay, size_t* bytes) {
  if (!bytes) return fail(LA_ERR_NULL_ARG, "bytes is NULL");
  la_status s = check_gated(B, T, Hq, Hkv, Dk, Dv, dtype);
  if (s != LA_OK) return s;
  const int64_t U = B * Hkv, G = Hq / Hkv;
  *bytes = 0;
  if (U > 0 && T > 1 && !by_token(per_dim_decay != 0, dtype, Dk, T))
    *bytes = delta_ws_bytes(U, Dk, plan_delta(U, G / head_tile(G), T));
  return ok();
}

LA_EXPORT la_status la_delta_forward(const void* q, const void* k, const void* v, const void* decay,
                                     int32_t per_dim_decay, const void* beta, int32_t beta_per_head,
                                     const float* past_state, float* present_state, void* out,
                                     int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t Dk,
                                     int64_t Dv, int32_t dtype, float scale, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  la_status s = check_gated(B, T, Hq, Hkv, Dk, Dv, dtype);
  if (s != LA_OK) return s;
  if (isnan(scale) || isinf(scale)) return fail(LA_ERR_BAD_ARG, "scale must be finite");
  const int64_t D = Dk, U = B * Hkv, G = Hq / Hkv;
  const int64_t esz = dtype_size(dtype);
  const bool per_dim = per_dim_decay != 0 && decay != nullptr;
  if (U > 0 && !present_state) return fail(LA_ERR_NULL_ARG, "present_state is required");
  const bool work = U > 0 && T > 0;
  if (work && (!q || !k || !v || !out || !beta))
    return fail(LA_ERR_NULL_ARG, "q, k, v, beta and out are required");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(past_state) ||
      !aligned16(present_state) || (per_dim && !aligned16(decay)))
    return fail(LA_ERR_BAD_ARG, "q, k, v, out, a per-dim decay and the states must be 16-byte aligned");
  const int64_t bh = beta_per_head ? Hkv : 1;
  const Range rq = range(q, B * T * Hq * D * esz), rk = range(k, B * T * Hkv * D * esz);
  const Range rv = range(v, B * T * Hkv * D * esz), ro = range(out, B * T * Hq * D * esz);
  const Range rg = range(decay, B * T * Hkv * (per_dim ? D : 1) * esz), rb = range(beta, B * T * bh * esz);
  const Range rpi = range(past_state, U * D * D * 4), rpo = range(present_state, U * D * D * 4);
  const Range ins[5] = {rq, rk, rv, rg, rb};
  for (const Range& i : ins)
    if (overlap(ro, i) || overlap(rpo, i)) return fail(LA_ERR_BAD_ARG, "an output overlaps an input");
  if (overlap(ro, rpi) || overlap(ro, rpo)) return fail(LA_ERR_BAD_ARG, "out overlaps a state buffer");
  if (overlap(rpo, rpi) && present_state != past_state)
    return fail(LA_ERR_BAD_ARG, "present_state may equal past_state exactly but not partially overlap it");
  if (U > (int64_t)1 << 31) return fail(LA_ERR_SHAPE, "too many (batch, kv head) units");
  if (workspace && workspace_bytes > 0) {
    if (!aligned16(workspace)) return fail(LA_ERR_BAD_ARG, "the workspace must be 16-byte aligned");
    const Range rw = range(workspace, (int64_t)workspace_bytes);
    for (const Range& i : ins)
      if (overlap(rw, i)) return fail(LA_ERR_BAD_ARG, "the workspace overlaps an input");
    if (overlap(rw, ro) || overlap(rw, rpi) || overlap(rw, rpo))
      return fail(LA_ERR_BAD_ARG, "the workspace overlaps out or a state buffer");
  }
  if (scale == 0.f) scale = 1.f / sqrtf((float)D);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (!work) {
    if (U > 0)
      e = past_state ? (present_state != past_state
                            ? la::launch_copy(present_state, past_state, U * D * D, st)
                            : hipSuccess)
                     : la::launch_fill_zero(present_state, U * D * D, st);
    return device_status(e, "la_delta_forward");
  }
  if (T == 1) {
    // one token: the streaming step (one read and one write of the state)
    la::GatedStepArgs g;
    memset(&g, 0, sizeof(g));
    g.q = q;
    g.k = k;
    g.v = v;
    g.decay = decay;
    g.s_in = past_state;
    g.s_out = present_state;
    g.out = out;
    g.Hkv = (int32_t)Hkv;
    g.units = (int32_t)U;
    g.per_dim = per_dim ? 1 : 0;
    g.scale = scale;
    g.beta = beta;
    g.beta_heads = (int32_t)bh;
    e = la::launch_delta_step(dtype, (int)D, (int)G, g, st);
    return device_status(e, "la_delta_forward (T = 1)");
  }
  if (by_token(per_dim, dtype, D, T)) {
    e = launch_by_token(q, k, v, decay, beta, bh, 1, past_state, present_state, out, B, T, Hq, Hkv, D, dtype,
                        scale, st);
    return device_status(e, "la_delta_forward (token by token)");
  }
  la::DeltaArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.decay = decay;
  a.beta = beta;
  a.out = out;
  a.s_in = past_state;
  a.s_out = present_state;
  a.T = (int32_t)T;
  a.Hq = (int32_t)Hq;
  a.Hkv = (int32_t)Hkv;
  a.units = (int32_t)U;
  a.beta_heads = (int32_t)bh;
  a.scale = scale;
  const int kind = decay == nullptr ? 0 : (per_dim ? 2 : 1);
  a.hsplit = (int32_t)(G / head_tile(G));
  a.nseg = 1;
  a.seg_len = (int32_t)T;
  a.s_in_u = D * D;
  a.s_out_u = D * D;
  const DeltaPlan p = plan_delta(U, a.hsplit, T);
  const size_t need = delta_ws_bytes(U, D, p);
  if (need == 0 || !workspace || workspace_bytes < need) {
    // one workgroup per (unit, head group) over the whole sequence; with the
    // state updated in place by several head groups, the groups that only read
    // it run first, then group 0, which also writes it
    if (a.hsplit > 1 && past_state && past_state == present_state) {
      la::DeltaArgs r = a;
      r.hg_first = 1;
      r.hg_count = a.hsplit - 1;
      e = la::launch_delta(dtype, (int)D, (int)head_tile(G), kind, r, st);
      r.hg_first = 0;
      r.hg_count = 1;
      if (e == hipSuccess) e = la::launch_delta(dtype, (int)D, (int)head_tile(G), kind, r, st);
    } else {
      e = la::launch_delta(dtype, (int)D, (int)head_tile(G), kind, a, st);
    }
    return device_status(e, "la_delta_forward");
  }
  // split over T: each segment's maps M (from S = I, zero values) and N (from
  // S = 0), the start states by composing them in order, then every segment
  // with outputs from its start state
  const int64_t E = D * D, nseg = p.nseg;
  float* Mw = (float*)workspace;
  float* Nw = Mw + U * (nseg - 1) * E;
  float* Sw = Nw + U * (nseg - 1) * E;
  float* I = Sw + U * nseg * E;
  e = la::launch_eye(I, (int)D, st);
  la::DeltaArgs m = a;
  m.out = nullptr;
  m.hsplit = 1;
  m.nseg = (int32_t)(nseg - 1);
  m.seg_len = (int32_t)p.seg_len;
  m.s_out_u = (nseg - 1) * E;
  m.s_out_s = E;
  m.s_out_all = 1;
  la::DeltaArgs n = m;
  m.v = nullptr;
  m.s_in = I;
  m.s_in_u = 0;
  m.s_in_s = 0;
  m.s_out = Mw;
  n.s_in = nullptr;
  n.s_out = Nw;
  if (e == hipSuccess) e = la::launch_delta(dtype, (int)D, 1, kind, m, st);
  if (e == hipSuccess) e = la::launch_delta(dtype, (int)D, 1, kind, n, st);
  if (e == hipSuccess) e = la::launch_delta_compose(Mw, Nw, past_state, Sw, (int)U, (int)nseg, (int)D, st);
  if (e == hipSuccess) {
    la::DeltaArgs o = a;
    o.nseg = (int32_t)nseg;
    o.seg_len = (int32_t)p.seg_len;
    o.s_in = Sw;
    o.s_in_u = nseg * E;
    o.s_in_s = E;
    e = la::launch_delta(dtype, (int)D, (int)head_tile(G), kind, o, st);
  }
  return device_status(e, "la_delta_forward (split)");
}

// ---------------------------------------------------------------------------
// causal backward

namespace {
struct BwdLayout {
  size_t den, fq, fk, v32, zc, rs, dnum, dden, qa, kc, vd, s0t, dstt, scratch, gws, total;
};
BwdLayout bwd_layout(int64_t B, int64_t T, int64_t H, int64_t D, int64_t esz, bool norm) {
  const size_t N = (size_t)(B * T * H * D), NT = (size_t)(B * T * H), SE = (size_t)(B * H * D * D);
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  BwdLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += al(bytes);
    return o;
  };
  L.den = take(norm ? NT * 4 : 0);
  L.fq = take(N * 4);
  L.fk = take(N * 4);
  L.v32 = take(N * 4);
  L.zc = take(norm ? N * 4 : 0);
  L.rs = take(norm ? N * 4 : 0);
  L.dnum = take(N * 4);
  L.dden = take(NT * 4);
  L.qa = take(N * 4);
  L.kc = take(N * 4);
  L.vd = take(N * 4);
  L.s0t = take(SE * 4);
  L.dstt = take(SE * 4);
  L.scratch = take(SE * 4);
  L.gws = take(gated_ws_bytes(B, T, H, D, false));
  L.total = off;
  return L;
}

// The chunk-parallel backward (16-bit inputs, head sizes 32 or 64): the
// forward segment states and the reverse gradient sums in slots (split
// sequences only), 1/den and dden per token (with the normaliser).
struct BwdChunkLayout {
  int64_t nseg, seg_len;
  size_t fs, fz, rs, rz, rden, dden, total;
};
BwdChunkLayout bwd_chunk_layout(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, bool norm) {
  const int64_t U = B * H;
  const CausalPlan p = plan_causal(U, T);
  BwdChunkLayout L;
  L.nseg = p.nseg;
  L.seg_len = p.seg_chunks * kChunk;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += al(bytes);
    return o;
  };
  const size_t slots = p.nseg > 1 ? (size_t)(U * p.nseg) : 0;
  L.fs = take(slots * Dk * Dv * 4);
  L.fz = take(norm ? slots * Dk * 4 : 0);
  L.rs = take(slots * Dk * Dv * 4);
  L.rz = take(norm ? slots * Dk * 4 : 0);
  L.rden = take(norm ? (size_t)(B * T * H) * 4 : 0);
  L.dden = take(norm ? (size_t)(B * T * H) * 4 : 0);
  L.total = off;
  return L;
}

// which backward runs: 1 chunk-parallel, 0 the recurrence-based one (head sizes
// equal), -1 none
int bwd_path(int32_t dtype, int64_t Dk, int64_t Dv) {
  if ((dtype == LA_DT_BF16 || dtype == LA_DT_F16) && (Dk == 32 || Dk == 64) && (Dv == 32 || Dv == 64)) return 1;
  return Dk == Dv ? 0 : -1;
}
}  // namespace

LA_EXPORT la_status la_backward_workspace_size(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                                               int32_t dtype, int32_t use_normalizer, size_t* bytes) {
  if (!bytes) return fail(LA_ERR_NULL_ARG, "bytes is NULL");
  la_status s = check_common(B, T, H, Dk, Dv, dtype);
  if (s != LA_OK) return s;
  const int path = bwd_path(dtype, Dk, Dv);
  if (path < 0)
    return fail(LA_ERR_UNSUPPORTED, "la_backward: Dk=%lld != Dv=%lld needs 16-bit inputs and head sizes 32 or 64",
                (long long)Dk, (long long)Dv);
  const bool norm = use_normalizer != 0;
  if (B * H == 0 || T == 0)
    *bytes = 0;
  else
    *bytes = path == 1 ? bwd_chunk_layout(B, T, H, Dk, Dv, norm).total
                       : bwd_layout(B, T, H, Dk, dtype_size(dtype), norm).total;
  return ok();
}

LA_EXPORT la_status la_backward(const void* q, const void* k, const void* v, const uint8_t* mask,
                                const float* state_in_kv, const float* state_in_k, const void* dout,
                                const float* dstate_out_kv, const float* dstate_out_k, int32_t feature_map,
                                int32_t use_normalizer, float eps, void* dq, void* dk, void* dv,
                                float* dstate_in_kv, float* dstate_in_k, int64_t B, int64_t T, int64_t H,
                                int64_t Dk, int64_t Dv, int32_t dtype, void* workspace,
                                size_t workspace_bytes, void* stream) {
  la_status s = check_common(B, T, H, Dk, Dv, dtype);
  if (s != LA_OK) return s;
  const int path = bwd_path(dtype, Dk, Dv);
  if (path < 0)
    return fail(LA_ERR_UNSUPPORTED, "la_backward: Dk=%lld != Dv=%lld needs 16-bit inputs and head sizes 32 or 64",
                (long long)Dk, (long long)Dv);
  if (feature_map != LA_FM_ELU_PLUS_ONE && feature_map != LA_FM_RELU_EPS)
    return fail(LA_ERR_BAD_ARG, "feature_map %d is not 0 (elu+1) or 1 (relu+eps)", feature_map);
  if (!(eps >= 0.f) || isinf(eps)) return fail(LA_ERR_BAD_ARG, "eps must be finite and >= 0");
  const bool norm = use_normalizer != 0;
  const int64_t D = Dk, U = B * H, SE = U * Dk * Dv;
  const int64_t esz = dtype_size(dtype);
  if (U == 0) return ok();
  if (!dstate_in_kv || (norm && !dstate_in_k))
    return fail(LA_ERR_NULL_ARG, "dstate_in (kv, and k with the normalizer) is required");
  if (norm) {
    if ((state_in_kv != nullptr) != (state_in_k != nullptr))
      return fail(LA_ERR_STATE, "normalized state_in needs both kv and k (or neither)");
    if ((dstate_out_kv != nullptr) != (dstate_out_k != nullptr))
      return fail(LA_ERR_STATE, "normalized dstate_out needs both kv and k (or neither)");
  } else if (state_in_k || dstate_out_k || dstate_in_k) {
    return fail(LA_ERR_STATE, "use_normalizer=0 carries only the kv state; k parts must be NULL");
  }
  const bool work = T > 0;
  if (work && (!q || !k || !v || !dout || !dq || !dk || !dv))
    return fail(LA_ERR_NULL_ARG, "q, k, v, dout, dq, dk and dv are required");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) ||
      !aligned16(dv) || !aligned16(state_in_kv) || !aligned16(state_in_k) || !aligned16(dstate_out_kv) ||
      !aligned16(dstate_out_k) || !aligned16(dstate_in_kv) || !aligned16(dstate_in_k) || !aligned16(workspace))
    return fail(LA_ERR_BAD_ARG, "q, k, v, dout, dq, dk, dv, the states and the workspace must be 16-byte aligned");
  const int64_t nbk = B * T * H * Dk * esz, nbv = B * T * H * Dv * esz;
  const size_t need = !work ? 0
                            : (path == 1 ? bwd_chunk_layout(B, T, H, Dk, Dv, norm).total
                                         : bwd_layout(B, T, H, D, esz, norm).total);
  const Range ins[9] = {range(q, nbk), range(k, nbk), range(v, nbv), range(dout, nbv), range(mask, B * T),
                        range(state_in_kv, SE * 4), range(state_in_k, U * Dk * 4),
                        range(dstate_out_kv, SE * 4), range(dstate_out_k, U * Dk * 4)};
  const Range outs[6] = {range(dq, nbk), range(dk, nbk), range(dv, nbv), range(dstate_in_kv, SE * 4),
                         range(dstate_in_k, U * Dk * 4), range(workspace, (int64_t)need)};
  for (int i = 0; i < 6; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return fail(LA_ERR_BAD_ARG, "an output or the workspace overlaps an input");
    for (int j = i + 1; j < 6; ++j)
      if (overlap(outs[i], outs[j])) return fail(LA_ERR_BAD_ARG, "outputs overlap each other or the workspace");
  }
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(LA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (!work) {
    e = dstate_out_kv ? la::launch_copy(dstate_in_kv, dstate_out_kv, SE, st) : la::launch_fill_zero(dstate_in_kv, SE, st);
    if (e == hipSuccess && norm)
      e = dstate_out_k ? la::launch_copy(dstate_in_k, dstate_out_k, U * D, st)
                       : la::launch_fill_zero(dstate_in_k, U * D, st);
    return device_status(e, "la_backward");
  }
  unsigned char* W = (unsigned char*)workspace;
  auto F = [&](size_t off) { return (float*)(W + off); };
  if (path == 1) {
    // chunk-parallel: forward segment states (split sequences), the forward
    // pass over every segment, the reverse prefix of its gradient sums, the
    // reverse pass
    const BwdChunkLayout C = bwd_chunk_layout(B, T, H, Dk, Dv, norm);
    const int64_t nseg = C.nseg, ZE = Dk;
    const bool fold = nseg <= la::kBwdFold;
    la::BwdChunkArgs c;
    memset(&c, 0, sizeof(c));
    c.q = q;
    c.k = k;
    c.v = v;
    c.dy = dout;
    c.mask = mask;
    c.rden = norm ? F(C.rden) : nullptr;
    c.dden = norm ? F(C.dden) : nullptr;
    c.dq = dq;
    c.dk = dk;
    c.dv = dv;
    c.T = (int32_t)T;
    c.H = (int32_t)H;
    c.nseg = (int32_t)nseg;
    c.seg_len = (int32_t)C.seg_len;
    c.fm = feature_map;
    c.eps = eps;
    if (nseg > 1) {
      // segments 0..nseg-2 -> slots 1..nseg-1, then the prefix (slot 0 = state_in)
      la::BwdChunkArgs ps = c;
      ps.nseg = (int32_t)(nseg - 1);
      ps.s_out = F(C.fs);
      ps.z_out = norm ? F(C.fz) : nullptr;
      ps.s_out_u = nseg * Dk * Dv;
      ps.s_out_s = Dk * Dv;
      ps.z_out_u = nseg * ZE;
      ps.z_out_s = ZE;
      e = la::launch_bwd_chunk(2, dtype, (int)Dk, (int)Dv, norm, ps, (int)(U * (nseg - 1)), st);
      // up to kBwdFold segments the passes add the slots themselves
      if (e == hipSuccess && !fold)
        e = la::launch_seg_prefix(F(C.fs), norm ? F(C.fz) : nullptr, state_in_kv, state_in_k, (int)U, (int)nseg,
                                  (int)Dk, (int)Dv, norm, st);
      if (e != hipSuccess) return device_status(e, "la_backward");
    }
    la::BwdChunkArgs c0 = c;
    c0.fold = fold ? 1 : 0;
    c0.s_init = state_in_kv;
    c0.z_init = norm ? state_in_k : nullptr;
    if (nseg > 1) {
      c0.s_in = F(C.fs);
      c0.z_in = norm ? F(C.fz) : nullptr;
      c0.s_in_u = nseg * Dk * Dv;
      c0.s_in_s = Dk * Dv;
      c0.z_in_u = nseg * ZE;
      c0.z_in_s = ZE;
      c0.s_out = F(C.rs);
      c0.z_out = norm ? F(C.rz) : nullptr;
      c0.s_out_u = nseg * Dk * Dv;
      c0.s_out_s = Dk * Dv;
      c0.z_out_u = nseg * ZE;
      c0.z_out_s = ZE;
    }
    e = la::launch_bwd_chunk(0, dtype, (int)Dk, (int)Dv, norm, c0, (int)(U * nseg), st);
    if (e == hipSuccess && nseg > 1 && !fold)
      e = la::launch_seg_prefix(F(C.rs), norm ? F(C.rz) : nullptr, dstate_out_kv, dstate_out_k, (int)U, (int)nseg,
                                (int)Dk, (int)Dv, norm, st);
    if (e != hipSuccess) return device_status(e, "la_backward");
    la::BwdChunkArgs c1 = c;
    c1.fold = fold ? 1 : 0;
    c1.s_init = dstate_out_kv;
    c1.z_init = norm ? dstate_out_k : nullptr;
    if (nseg > 1) {
      c1.s_in = F(C.rs);
      c1.z_in = norm ? F(C.rz) : nullptr;
      c1.s_in_u = nseg * Dk * Dv;
      c1.s_in_s = Dk * Dv;
      c1.z_in_u = nseg * ZE;
      c1.z_in_s = ZE;
    }
    c1.s_out = dstate_in_kv;
    c1.z_out = dstate_in_k;
    c1.s_out_u = Dk * Dv;
    c1.z_out_u = ZE;
    e = la::launch_bwd_chunk(1, dtype, (int)Dk, (int)Dv, norm, c1, (int)(U * nseg), st);
    return device_status(e, "la_backward");
  }
  // the recurrence-based backward (fp32 inputs, head size 128)
  const BwdLayout L = bwd_layout(B, T, H, D, esz, norm);
  la::BwdArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.dy = dout;
  a.mask = mask;
  a.den = norm ? F(L.den) : nullptr;
  a.fq = F(L.fq);
  a.fk = F(L.fk);
  a.v32 = F(L.v32);
  a.dnum = F(L.dnum);
  a.dden = F(L.dden);
  a.qa = F(L.qa);
  a.kc = F(L.kc);
  a.vd = F(L.vd);
  a.zc = norm ? F(L.zc) : nullptr;
  a.rs = norm ? F(L.rs) : nullptr;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.B = (int32_t)B;
  a.T = (int32_t)T;
  a.H = (int32_t)H;
  a.D = (int32_t)D;
  a.fm = feature_map;
  a.eps = eps;
  // 1. phi(q), phi(k), v; 2. z_i; 3. den and dnum
  e = la::launch_bwd_prep(dtype, a, st);
  if (e == hipSuccess && norm)
    e = la::launch_bwd_scan(F(L.fk), nullptr, state_in_k, F(L.zc), nullptr, (int)U, (int)T, (int)H, (int)D, 0, st);
  if (e == hipSuccess) e = la::launch_bwd_dnum(dtype, a, st);
  if (e == hipSuccess && state_in_kv) e = la::launch_bwd_transpose(state_in_kv, F(L.s0t), U, (int)D, st);
  if (e == hipSuccess && dstate_out_kv) e = la::launch_bwd_transpose(dstate_out_kv, F(L.dstt), U, (int)D, st);
  if (e != hipSuccess) return device_status(e, "la_backward");
  // 4. qa_i = S_i dnum_i (the first linear-rule recurrence, fp32, scale 1)
  void* gw = W + L.gws;
  const size_t gwb = L.total - L.gws;
  s = la_gated_forward(F(L.dnum), F(L.v32), F(L.fk), nullptr, 0, state_in_kv ? F(L.s0t) : nullptr,
                       F(L.scratch), F(L.qa), B, T, H, H, D, D, LA_DT_F32, 1.f, gw, gwb, stream);
  if (s != LA_OK) return s;
  // 5. dden from qa, then dz_0 and the reverse sums dz_T + sum_{i>=j} phi_q_i dden_i
  if (norm) {
    e = la::launch_bwd_dden(a, st);
    if (e == hipSuccess)
      e = la::launch_bwd_scan(F(L.fq), F(L.dden), dstate_out_k, F(L.rs), dstate_in_k, (int)U, (int)T, (int)H,
                              (int)D, 1, st);
  } else {
    e = la::launch_fill_zero(F(L.dden), B * T * H, st);
  }
  if (e != hipSuccess) return device_status(e, "la_backward");
  // 6. the reversed-time recurrences, run backwards over the time-ordered buffers
  s = gated_forward(F(L.v32), F(L.dnum), F(L.fq), nullptr, 0, dstate_out_kv ? F(L.dstt) : nullptr,
                    F(L.scratch), F(L.kc), B, T, H, H, D, D, LA_DT_F32, 1.f, gw, gwb, stream, 1);
  if (s != LA_OK) return s;
  s = gated_forward(F(L.fk), F(L.fq), F(L.dnum), nullptr, 0, dstate_out_kv, dstate_in_kv, F(L.vd), B, T, H, H, D,
                    D, LA_DT_F32, 1.f, gw, gwb, stream, 1);
  if (s != LA_OK) return s;
  // 7. dq, dk, dv
  e = la::launch_bwd_finish(dtype, a, st);
  return device_status(e, "la_backward");
}
