// Internal interface between the C-ABI front end (la_api.cpp) and the kernel
// translation units.  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

// Arguments of the chunk-parallel kernel (la_chunk.hip).  A workgroup handles
// unit u = (b,h) and segment s = seg_first + blockIdx % seg_count, i.e. chunks
// [s*seg_chunks, min((s+1)*seg_chunks, nchunks)) of 64 tokens.
struct ChunkArgs {
  const void* q;
  const void* k;
  const void* v;
  const uint8_t* mask;  // (B,T) or null
  void* out;
  // initial state of the segment (null = zeros): s_in + u*s_in_u + s*s_in_s.
  // With fold (causal mode) s_in holds the unprefixed segment sums in slots
  // 1 .. nseg-1, and segment s starts from s_init + u*s_init_u (z_init + u*z_init_u;
  // null = zeros) plus slots 1 .. s, added in slot order (s < kChunkFold)
  const float* s_in;
  const float* z_in;
  int64_t s_in_u, s_in_s, z_in_u, z_in_s;
  const float* s_init;
  const float* z_init;
  int64_t s_init_u, z_init_u;
  int32_t fold;
  // state written at the end (causal: by the last segment only; state mode:
  // slot s + out_slot_off of unit u)
  float* s_out;
  float* z_out;
  int64_t s_out_u, s_out_s, z_out_u, z_out_s;
  int32_t out_slot_off;
  int32_t T, H;
  int32_t seg_count, seg_first, seg_chunks, nseg_total;
  // 0 or 1: segment s is the seg_chunks consecutive chunks from s*seg_chunks.
  // n > 1 (the state mode of a non-causal reduction, whose sum does not depend
  // on order): segment s takes chunks s, s+n, s+2n, ..., so masked tails are
  // spread over all segments of a unit
  int32_t chunk_step;
  float eps;
  // head sizes when they differ (Dk != Dv): the kernel runs at the larger, D,
  // with the smaller side zero-padded (feature map of padded q/k dims 0); q, k
  // rows are (.., H, dk), v, out rows (.., H, dv), states dk x dv (+ dk).
  // 0 = both D.
  int32_t dk, dv;
};

enum { kModeCausal = 0, kModeState = 1, kModeRerun = 2 };
// I/O element type codes of the launchers (the values of la_dtype)
enum { kIoF32 = 0, kIoBF16 = 1, kIoF16 = 2 };

// segment counts up to which the causal pass at head sizes up to 64 forms its
// segment states itself (fold) instead of a prefix pass over the slots
constexpr int kChunkFold = 8;
hipError_t launch_chunk(int mode, int io, int D, int fm, int norm, const ChunkArgs& a, int grid,
                        hipStream_t st);
// slots of dk x dv (+ dk with the normaliser) floats
hipError_t launch_seg_prefix(float* ws_s, float* ws_z, const float* s_in, const float* z_in, int U,
                             int nseg, int dk, int dv, int norm, hipStream_t st);
hipError_t launch_seg_sum(float* ws_s, float* ws_z, int U, int nseg, int dk, int dv, int norm,
                          hipStream_t st);

// Non-causal readout with a fixed summed state (la_apply.hip).  Workgroup
// blockIdx of unit u = blockIdx / seg_count handles the unit's 16-row query
// blocks sg, sg + seg_count, ... (sg = blockIdx % seg_count); every wave of it
// takes at most 16 of them, so seg_count must be apply_groups_per_unit(U, T).
struct ApplyArgs {
  const void* q;        // (B,T,H,D)
  const uint8_t* mask;  // (B,T) or null
  void* out;            // (B,T,H,D)
  const float* s;       // summed S of unit u at s + u*s_u, [dk][dv]
  const float* z;       // summed Z of unit u at z + u*z_u (with the normaliser)
  int64_t s_u, z_u;
  int32_t T, H;
  int32_t seg_count;
  float eps;
  int32_t dk, dv;  // as ChunkArgs (0 = both D); s is dk x dv, z dk
};
int apply_groups_per_unit(int64_t U, int64_t T);
hipError_t launch_apply(int io, int D, int fm, int norm, const ApplyArgs& a, int grid,
                        hipStream_t st);

// T == 1 decode step (la_decode.hip).  q,k: (B,H,Dk); v,out: (B,H,Dv); state
// (B,H,Dk,Dv)+(B,H,Dk).
struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const uint8_t* mask;  // (B) or null
  const float* s_in;
  const float* z_in;
  float* s_out;
  float* z_out;
  void* out;
  int32_t H;
  int32_t units;  // B*H
  float eps;
};
hipError_t launch_decode(int io, int Dk, int Dv, int fm, int norm, const DecodeArgs& a, int units,
                         hipStream_t st);

// Zero fill (la_decode.hip).
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st);
hipError_t launch_copy(float* dst, const float* src, int64_t n, hipStream_t st);

// Gated GQA recurrence (la_gated.hip).
struct GatedArgs {
  const void* q;      // (B,T,Hq*D)
  const void* k;      // (B,T,Hkv*D)
  const void* v;      // (B,T,Hkv*D)
  const void* decay;  // (B,T,Hkv), or (B,T,Hkv*D) for the per-dim kernel, or null
  void* out;          // (B,T,Hq*D)
  const float* s_in;  // initial state of the segment, s_in + u*s_in_u + s*s_in_s (null = zeros)
  int64_t s_in_u, s_in_s;
  float* s_out;       // final/partial state, see launch_gated
  int64_t s_out_u, s_out_s;
  float* a_out;       // state mode: per (unit, slot) total decay factor (per (unit, slot, dk): per-dim)
  int32_t out_slot_off;
  int32_t T, Hq, Hkv;
  int32_t seg_count, seg_first, seg_chunks, nseg_total;
  float scale;
  // 1: run in reversed time, token t of the recurrence being row T-1-t of q,
  // k, v, the decay and out (la_gated.hip only; the per-dim kernel takes 0)
  int32_t reverse;
  // query-head groups (0 or 1: one): a kv head's Hq/Hkv query heads are split
  // over hsplit workgroups of G heads each (the launcher's G), which all run
  // the unit's recurrence; group 0 writes the state.  A launch runs groups
  // hg_first .. hg_first + hg_count - 1 (hg_count 0: all), blockIdx = (unit-
  // segment index) * hg_count + group - hg_first.  The state pass (kModeState)
  // takes 1.
  int32_t hsplit, hg_first, hg_count;
  // per-dim kernel: one int per (unit, segment), u * nseg_total + s.  The
  // output pass (kModeCausal) stores 1 where the segment's decays are too
  // strong for its chunk form (and then leaves its state unwritten), else 0;
  // the re-evaluation launch (kModeRerun, same grid and groups) redoes those
  // segments token by token, outputs and state.
  int32_t* flags;
};
hipError_t launch_gated(int mode, int io, int D, int G, const GatedArgs& a, int grid,
                        hipStream_t st);

// Delta rules (la_delta.hip): one workgroup per (batch, kv head) unit over the
// whole sequence.
struct DeltaArgs {
  const void* q;      // (B,T,Hq*D)
  const void* k;      // (B,T,Hkv*D)
  const void* v;      // (B,T,Hkv*D)
  const void* decay;  // null, (B,T,Hkv) or (B,T,Hkv*D) per the decay kind
  const void* beta;   // (B,T,beta_heads)
  void* out;          // (B,T,Hq*D)
  const float* s_in;  // (B*Hkv,D,D) or null (zeros)
  float* s_out;       // (B*Hkv,D,D)
  int32_t T, Hq, Hkv, units, beta_heads;
  float scale;
  // query-head groups, as GatedArgs::hsplit, hg_first and hg_count
  // (grid = units * nseg * hg_count, hg_count 0: hsplit)
  int32_t hsplit, hg_first, hg_count;
  // Split over T: segment s of nseg (0 or 1: one) covers tokens
  // [s * seg_len, min((s + 1) * seg_len, T)) (seg_len 0: T; a single segment
  // may be shorter than the sequence); blockIdx = (u * nseg + s) * hg_count
  // + group.  The segment starts from s_in + u * s_in_u + s * s_in_s (null:
  // zeros) and writes its final state to s_out + u * s_out_u + s * s_out_s when
  // s_out_all, else only the last segment does.  v null: the values are zero;
  // out null: no outputs.
  int32_t nseg, seg_len, s_out_all;
  int64_t s_in_u, s_in_s, s_out_u, s_out_s;
};
// decay_kind: 0 none ("delta"), 1 per kv head, 2 per key dim.  fp32 at head
// size 128 is not available (LDS).
hipError_t launch_delta(int io, int D, int G, int decay_kind, const DeltaArgs& a, hipStream_t st);
// Segment start states of a split delta-rule sequence (la_delta.hip): for each
// of `units` units, start(0) = past (null: zeros) and start(s + 1) = M_s start(s)
// + N_s, with M_s, N_s, start(s) the D x D slots s of the unit (nseg - 1 of M
// and N, nseg of start); slot strides D * D, unit strides (nseg - 1) * D * D for
// M, N and nseg * D * D for start.
hipError_t launch_delta_compose(const float* M, const float* N, const float* past, float* start, int units,
                                int nseg, int D, hipStream_t st);
// The D x D identity.
hipError_t launch_eye(float* p, int D, hipStream_t st);

// Causal backward (la_backward.hip): buffers are (B,T,H,D) fp32 unless noted.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dy;       // (I/O type)
  const uint8_t* mask;  // (B,T) or null
  float* den;           // (B,T,H) denominators (formed by the dnum kernel), or null without the normalizer
  float* fq;
  float* fk;
  float* v32;
  float* dnum;
  float* dden;          // (B,T,H)
  const float* qa;      // S_i dnum_i
  const float* kc;      // sum_{i>=j} phi_q_i (v_j . dnum_i) + dS_T v_j
  const float* vd;      // dv
  const float* zc;      // z_i (normalized), or null
  const float* rs;      // dz_T + sum_{i>=j} phi_q_i dden_i (normalized), or null
  void* dq;
  void* dk;
  void* dv;
  int32_t B, T, H, D, fm;
  float eps;
};
hipError_t launch_bwd_prep(int io, const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_scan(const float* x, const float* w, const float* init, float* out, float* total, int U,
                           int T, int H, int D, int reverse, hipStream_t st);
hipError_t launch_bwd_dnum(int io, const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_dden(const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_finish(int io, const BwdArgs& a, hipStream_t st);
hipError_t launch_bwd_transpose(const float* in, float* out, int64_t U, int D, hipStream_t st);

// Chunk-parallel causal backward for 16-bit inputs at head sizes Dk, Dv in
// {32, 64} (la_bwd_chunk.hip).  Workgroup blockIdx covers unit u = blockIdx /
// nseg and tokens [s*seg_len, min((s+1)*seg_len, T)) of segment s = blockIdx %
// nseg (seg_len a multiple of 32).
struct BwdChunkArgs {
  const void* q;        // (B,T,H,Dk)
  const void* k;        // (B,T,H,Dk)
  const void* v;        // (B,T,H,Dv)
  const void* dy;       // (B,T,H,Dv), passes 0 and 1
  const uint8_t* mask;  // (B,T) or null
  // pass 0: forward state at the start of segment s, s_in + u*s_in_u + s*s_in_s
  // ([dk][dv], z [dk]; null = zeros).  pass 1: the gradient sums of the tokens
  // after segment s, at slot nseg - 1 - s (null = zeros).  With fold set the
  // slots are not prefixed: the state is s_init + u*Dk*Dv (z_init + u*Dk; null
  // = zeros) plus slots 1 .. R of s_in (R = s in pass 0, nseg - 1 - s in pass
  // 1, at most kBwdFold - 1), added in slot order
  const float* s_in;
  const float* z_in;
  int64_t s_in_u, s_in_s, z_in_u, z_in_s;
  const float* s_init;
  const float* z_init;
  int32_t fold;
  // pass 0: segment s >= 1 writes its sum of phi_q dnum^T (phi_q dden) to slot
  // nseg - s; pass 1: segment 0 writes dS_0, dz_0 at s_out + u*s_out_u
  float* s_out;
  float* z_out;
  int64_t s_out_u, s_out_s, z_out_u, z_out_s;
  // (B,T,H) fp32 with the normaliser: 1/den_i at valid tokens, 0 elsewhere;
  // written by pass 0, read by pass 1, which rebuilds dnum_i = dy_i / den_i
  // (the same fp32 product pass 0 forms)
  float* rden;
  float* dden;  // (B,T,H) fp32 (with the normaliser)
  void* dq;     // pass 0
  void* dk;     // pass 1
  void* dv;     // pass 1
  int32_t T, H, nseg, seg_len;
  int32_t fm;
  float eps;
};
// io: bf16 or fp16; Dk, Dv: 32 or 64 each.  pass 0: forward over each
// segment (dq, 1/den, dden, segment sums); pass 1: reverse (dk, dv, dS_0,
// dz_0); pass 2: the forward state's sum over segment s = blockIdx % nseg of
// each unit into slot s + 1 of s_out / z_out (strides s_out_u, s_out_s).
// segment counts up to which the chunk backward forms its segment states itself
// (fold) instead of a prefix pass over the slots
constexpr int kBwdFold = 8;
hipError_t launch_bwd_chunk(int pass, int io, int Dk, int Dv, int norm, const BwdChunkArgs& a, int grid,
                            hipStream_t st);

// T == 1 step of the gated recurrence (la_decode.hip).
struct GatedStepArgs {
  const void* q;      // (B, Hq*D)
  const void* k;      // (B, Hkv*D)
  const void* v;      // (B, Hkv*D)
  const void* decay;  // (B, Hkv), or (B, Hkv*D) with per_dim, or null
  const float* s_in;  // (B*Hkv, D, D) or null (zeros)
  float* s_out;       // (B*Hkv, D, D), may equal s_in
  void* out;          // (B, Hq*D)
  int32_t Hkv;
  int32_t units;  // B*Hkv
  int32_t per_dim;
  float scale;
  // delta rules only: beta (B, beta_heads), beta_heads = Hkv or 1 (shared)
  const void* beta;
  int32_t beta_heads;
  // query heads per kv head (0: the launcher's G); more than 8, or a count that
  // is not a power of two, runs the readout in passes of the largest of 8, 4,
  // 2, 1 that divides it
  int32_t heads;
  // rows per batch of q, k, v, the decay, beta and out: 0 or 1 for (B, ...)
  // tensors; T when the pointers sit at token t of (B, T, ...) tensors
  int32_t batch_rows;
};
hipError_t launch_gated_step(int io, int D, int G, const GatedStepArgs& a, hipStream_t st);
// T == 1 step of the delta rules (la_decode.hip): decay null ("delta"), per kv
// head, or per key dim (per_dim)
hipError_t launch_delta_step(int io, int D, int G, const GatedStepArgs& a, hipStream_t st);
hipError_t launch_gated_prefix(float* ws_s, const float* ws_a, const float* s_in, int U, int nseg,
                               int D, int per_dim, hipStream_t st);
// Per-key-dim decay (la_gated_pd.hip): the same arguments and modes as
// launch_gated, plus kModeRerun after each output pass (flags required in both);
// fp32 at head size 128 is not available (LDS).
hipError_t launch_gated_pd(int mode, int io, int D, int G, const GatedArgs& a, int grid, hipStream_t st);

// Whole-sequence token-by-token recurrence (la_recur.hip), one workgroup per
// (batch, kv head) unit, query-head group and group of 32 state columns; head
// size 128.
struct RecurArgs {
  const void* q;      // (B,T,Hq*D)
  const void* k;      // (B,T,Hkv*D)
  const void* v;      // (B,T,Hkv*D)
  const void* decay;  // null, (B,T,Hkv) or (B,T,Hkv*D) per the decay kind
  const void* beta;   // delta rule: (B,T,beta_heads)
  void* out;          // (B,T,Hq*D)
  const float* s_in;  // (B*Hkv,D,D) or null (zeros)
  float* s_out;       // (B*Hkv,D,D)
  int32_t T, Hq, Hkv, units, beta_heads, hsplit;
  float scale;
  int32_t hg_first, hg_count;  // query-head groups of one launch (set by launch_recur)
};
// decay_kind: 0 none, 1 per kv head, 2 per key dim; delta: the delta rule;
// G: query heads per workgroup (1, 2, 4, 8; hsplit groups of them per unit)
hipError_t launch_recur(int io, int D, int G, int decay_kind, int delta, const RecurArgs& a, hipStream_t st);

}  // namespace la
