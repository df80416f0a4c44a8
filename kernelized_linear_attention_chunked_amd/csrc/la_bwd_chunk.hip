// Chunk-parallel causal backward for 16-bit inputs (bf16, fp16) at head sizes
// Dk, Dv in {32, 64}: the gradients of the normalized causal recurrence of
// "[Feature] LinearAttention layer for Keras" ("Mathematical definition /
// Causal"; "Stability" and "Acceptance" ask for the gradients and their
// float64 checks).  Per (batch, head) unit, with phi_q = phi(q), phi_k = phi(k)
// (0 at invalid tokens), S_i, z_i the running sums through token i, and
// num_i = S_i^T phi_q_i, den_i = phi_q_i . z_i + eps, y_i = num_i / den_i:
//   dnum_i = m_i dy_i / den_i,  dden_i = -dnum_i . y_i     (normalized; else dnum_i = m_i dy_i, dden_i = 0)
//   B_ij   = dnum_i . v_j + dden_i                          (j <= i)
//   dphi_q_i = sum_{j<=i} B_ij phi_k_j + S_prev dnum_i + dden_i z_prev
//   dphi_k_j = sum_{i>=j} B_ij phi_q_i + dS_next v_j + dz_next
//   dv_j     = sum_{i>=j} (phi_q_i . phi_k_j) dnum_i + dS_next^T phi_k_j
//   dS_0 = dS_T + sum_i phi_q_i dnum_i^T,  dz_0 = dz_T + sum_i phi_q_i dden_i,
// where within a chunk S_prev, z_prev are the sums before it and dS_next,
// dz_next the gradient sums of the tokens after it (dS_T, dz_T included).
//
// A sequence is cut into segments (the forward's causal split):
//   bwd_state_kernel sums phi_k v^T (phi_k) over each segment but the last,
//                   and a prefix over those sums gives each segment its
//                   forward state at the start;
//   bwd_fwd_kernel  runs each segment forward in 32-token chunks with S, z in
//                   registers: dq, dnum and dden per token (1/den and dden to
//                   the workspace), and the segment's sum of phi_q dnum^T,
//                   phi_q dden;
//   (a prefix over those sums, in reverse segment order, gives each segment
//   its dS_next, dz_next at the segment end)
//   bwd_rev_kernel  runs each segment backwards with dS, dz in registers: dk,
//                   dv, and dS_0, dz_0 from the first segment; it forms dnum
//                   again from dy and 1/den (the same fp32 product), which
//                   moves 4 bytes per token instead of Dv fp32 values.
//
// Precision: the gradients cancel strongly (dden_i removes the dnum-weighted
// mean of the values from every B_ij, and the state terms carry the same
// offset), so a single bf16 rounding of any operand costs up to ~1e-1 relative
// error.  Every operand is therefore fed as bf16 hi + lo parts (hi = x rounded,
// lo = the remainder rounded) and every product takes hi*hi + hi*lo + lo*hi,
// about 16 significant bits; only operands that are exact in bf16 (the values
// of bf16 inputs, the ones of the normaliser rows) go as one part.
//
// Layout (8 wavefronts, one workgroup per (unit, segment)): every matrix a
// product contracts over sits in LDS with its contraction index contiguous,
// hi part then lo part, in unpadded rows whose 16-byte blocks are XOR-swizzled
// by a function of the row (ro, to below).  A product
// C += A B^T takes A's rows from one matrix and B's from another (see
// la_device.hpp for the MFMA lane layout).  The intra-chunk scores feed the
// next product straight from registers: a pair of score tiles whose A rows are
// the keys (queries) 8(r/4) + 4 odd + r%4 leaves lane group lg holding keys
// (queries) 8lg..8lg+7 of one column, which is the operand layout of a
// 32-wide contraction over them.
#include <type_traits>

#include "la_device.hpp"
#include "la_launch.hpp"

namespace la {
namespace {

constexpr int kBC = 32;        // tokens per chunk
constexpr int kBW = 8;         // wavefronts per workgroup
constexpr int kBT = 64 * kBW;  // threads

__device__ __forceinline__ void mm(f32x4_t& c, const u32x4_t& a, const u32x4_t& b) { Op<uint16_t>::mma(c, a, b); }
// (ah + al)(bh + bl) without the lo*lo term
__device__ __forceinline__ void mm3(f32x4_t& c, const u32x4_t& ah, const u32x4_t& al, const u32x4_t& bh,
                                    const u32x4_t& bl) {
  mm(c, ah, bh);
  mm(c, ah, bl);
  mm(c, al, bh);
}
// bf16 hi and lo parts of x (16-bit patterns)
__device__ __forceinline__ void split1(float x, uint32_t& h, uint32_t& lo) {
  h = f32_to_bf16_bits(x);
  lo = f32_to_bf16_bits(x - __uint_as_float(h << 16));
}
// hi and lo words of a pair (first value in bits 0..15)
__device__ __forceinline__ u32x2_t split2(float x0, float x1) {
  const uint32_t h = pack_bf16x2(x0, x1);
  return u32x2_t{h, pack_bf16x2(x0 - __uint_as_float(h << 16), x1 - __uint_as_float(h & 0xffff0000u))};
}
// a score tile pair (rows 8lg + 4odd + q of column lr) as operand words over
// the 8 rows 8lg .. 8lg+7
__device__ __forceinline__ void pair_operand(const f32x4_t (&at)[2], u32x4_t& h, u32x4_t& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) { const u32x2_t t2_ = split2(at[e >> 1][2 * (e & 1)], at[e >> 1][2 * (e & 1) + 1]); h[e] = t2_[0]; lo[e] = t2_[1]; }
}
// derivative of phi: elu(x)+1 -> 1 (x > 0) or exp(x); relu(x)+eps -> 1 (x > 0) or 0
__device__ __forceinline__ float dphi_rt(float x, bool elu) {
  return x > 0.f ? 1.f : (elu ? __expf(x) : 0.f);
}
// Range-checked buffer access: a resource of `bytes` bytes from `base`; loads
// past the range return 0 and stores past it are dropped, so every access of a
// chunk's tokens is issued unconditionally (a load or store under a branch
// would make the wait for an earlier load cover every access issued after it).
// Offsets are in bytes.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kDrop = 0x80000000u;  // past every range: the store is dropped
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t bload16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ u32x2_t bload8(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t bload4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bload1(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}
__device__ __forceinline__ void bstore16(rsrc_t r, uint32_t off, const u32x4_t& v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}
__device__ __forceinline__ void bstore8(rsrc_t r, uint32_t off, const u32x2_t& v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}
__device__ __forceinline__ void bstore4(rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
}
// four fp32 results as the I/O type
template <typename IT>
__device__ __forceinline__ u32x2_t pack4(float a, float b, float c, float d) {
  return u32x2_t{Io<IT>::pack2(a, b), Io<IT>::pack2(c, d)};
}
// the I/O value in half e of word w
template <typename IT>
__device__ __forceinline__ float io_at(uint32_t w, int e) {
  return Io<IT>::to_f32(e ? w >> 16 : w & 0xffffu);
}

// the two bf16 halves of word w as fp32 (element e of a 16-bit pair)
__device__ __forceinline__ float bf_at(uint32_t w, int e) {
  return __uint_as_float(e ? (w & 0xffff0000u) : (w << 16));
}

// Staging of two tokens' 8 values: phi applied (PHI), zeroed where the token
// is not ok, and split into bf16 hi and lo words along the row (element 2i in
// the low half of word i).
template <int FM, bool PHI>
__device__ __forceinline__ void split_rows(float (&f)[2][8], bool ok0, bool ok1, float eps, u32x4_t (&h)[2],
                                           u32x4_t (&lo)[2]) {
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const bool ok = n ? ok1 : ok0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = PHI ? phi<FM>(f[n][e], eps) : f[n][e];
      f[n][e] = ok ? x : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x2_t t = split2(f[n][2 * i], f[n][2 * i + 1]);
      h[n][i] = t[0];
      lo[n][i] = t[1];
    }
  }
}
// the transposed word of row element e from the row words of token a (low
// half) and token b (high half)
__device__ __forceinline__ uint32_t tword(const u32x4_t& a, const u32x4_t& b, int e) {
  return __builtin_amdgcn_perm(b[e >> 1], a[e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
}

// LDS tiles.  Row tiles hold N = 32 or 64 elements per row (a token's q, k, v
// or dnum, or a row of S^T or dS^T); token tiles hold the 32 tokens of a chunk
// per row (phi(Q)^T, phi(K)^T, V^T, dnum^T).  Rows are unpadded and their
// 16-byte blocks are XORed by a function of the row, chosen with a model of
// the gfx950 LDS (64 banks of 4 bytes; a 16-byte read serves lanes 0-7 with
// 24-31, 8-23, 32-39 with 56-63 and 40-55 in one cycle each, other accesses 32
// lanes at a time) so that the operand reads, both the row reads (row = lane
// % 16) and the permuted score rows 8(r/4) + 4 odd + r%4, are conflict-free;
// padding rows by one block made every one of them two-way.
template <int NB>
__device__ __forceinline__ int rsw(int r) {
  if constexpr (NB == 8)
    return ((r >> 1) & 7) ^ (((r >> 4) & 1) << 1);
  else
    return (r >> 2) & 3;
}
__device__ __forceinline__ int tsw(int r) { return ((((r >> 2) ^ (r >> 4)) & 1) << 1) ^ ((r >> 5) & 1); }
// element offset of (row r, column c) in a row tile of N elements per row
template <int N>
__device__ __forceinline__ int ro(int r, int c) {
  constexpr int NB = N / 8;
  return r * N + ((((c >> 3) ^ rsw<NB>(r)) & (NB - 1)) << 3) + (c & 7);
}
// element offset of (row r, token t) in a token tile
__device__ __forceinline__ int to(int r, int t) { return r * kBC + ((((t >> 3) ^ tsw(r)) & 3) << 3) + (t & 7); }
// column c of rows r0 .. r0+7 (r0 a multiple of 8) of a row tile as one MFMA
// operand (the tile read transposed): within the 8 rows the swizzle changes by
// a constant per row
template <int N>
__device__ __forceinline__ u32x4_t gather8(const uint16_t* tile, int r0, int c) {
  constexpr int NB = N / 8;
  const int s0 = rsw<NB>(r0), cb = c >> 3, ce = c & 7;
  u32x4_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e0 = 2 * i, e1 = 2 * i + 1;
    const int d0 = NB == 8 ? (e0 >> 1) : (e0 >> 2), d1 = NB == 8 ? (e1 >> 1) : (e1 >> 2);
    const uint32_t x0 = tile[(r0 + e0) * N + (((cb ^ s0 ^ d0) & (NB - 1)) << 3) + ce];
    const uint32_t x1 = tile[(r0 + e1) * N + (((cb ^ s0 ^ d1) & (NB - 1)) << 3) + ce];
    r[i] = x0 | (x1 << 16);
  }
  return r;
}

// Staging item of a thread: two consecutive tokens (2p, 2p+1) of one 16-byte
// column block (8 elements) of input matrix m.  The matrices take consecutive
// thread ranges of sizes N0, N1, N2, N3 (each a multiple of 64, so that every
// wave stages one matrix), with B0.. blocks per token row.
struct Item {
  int m, p, cb;
  bool on;
};
template <int N0, int B0, int N1, int B1, int N2, int B2, int N3 = 0, int B3 = 1>
__device__ __forceinline__ Item make_item(int tid) {
  static_assert(N0 % 64 == 0 && N1 % 64 == 0 && N2 % 64 == 0 && N3 % 64 == 0, "wave-uniform matrices");
  // the matrix and whether the wave stages at all are the same in every lane
  const int wt = __builtin_amdgcn_readfirstlane(tid & ~63);
  const int m = wt < N0 ? 0 : (wt < N0 + N1 ? 1 : (wt < N0 + N1 + N2 ? 2 : 3));
  const bool on = wt < N0 + N1 + N2 + N3;
  const int r = tid - (m == 0 ? 0 : (m == 1 ? N0 : (m == 2 ? N0 + N1 : N0 + N1 + N2)));
  const int bl = m == 0 ? B0 : (m == 1 ? B1 : (m == 2 ? B2 : B3));
  return on ? Item{m, r / bl, r % bl, true} : Item{m, 0, 0, false};
}

// The state a pass starts a segment from (element [d][col] of S, or of z with
// col < 0): slot `slot` of the prefixed slots, or with a.fold the initial
// state plus the unprefixed slots 1 .. R in slot order (the prefix pass's sum,
// with every slot's loads issued before the adds).
template <int DK, int DV, bool NORM>
struct StartState {
  const float *s0, *z0, *sl, *zl;
  int64_t ss, zs;
  int R;
  __device__ StartState(const BwdChunkArgs& a, int u, int slot, int R_) {
    if (a.fold) {
      s0 = a.s_init ? a.s_init + (int64_t)u * DK * DV : nullptr;
      z0 = (NORM && a.z_init) ? a.z_init + (int64_t)u * DK : nullptr;
      sl = a.s_in ? a.s_in + u * a.s_in_u : nullptr;
      zl = (NORM && a.z_in) ? a.z_in + u * a.z_in_u : nullptr;
      R = sl ? R_ : 0;
    } else {
      s0 = a.s_in ? a.s_in + u * a.s_in_u + slot * a.s_in_s : nullptr;
      z0 = (NORM && a.z_in) ? a.z_in + u * a.z_in_u + slot * a.z_in_s : nullptr;
      sl = zl = nullptr;
      R = 0;
    }
    ss = a.s_in_s;
    zs = a.z_in_s;
  }
  __device__ float at(int d, int col) const {
    const float* b = col >= 0 ? s0 : z0;
    const float* l = col >= 0 ? sl : zl;
    const int64_t o = col >= 0 ? (int64_t)d * DV + col : d;
    const int64_t st = col >= 0 ? ss : zs;
    float y[kBwdFold - 1];
#pragma unroll
    for (int r = 1; r < kBwdFold; ++r) y[r - 1] = r <= R ? l[r * st + o] : 0.f;
    float x = b ? b[o] : 0.f;
#pragma unroll
    for (int r = 1; r < kBwdFold; ++r)
      if (r <= R) x += y[r - 1];
    return x;
  }
};

// ---------------------------------------------------------------------------
// Forward pass of the backward: LDS layout in 16-bit elements.
template <int DK, int DV, bool NORM, bool VLO>
struct FwdLds {
  static constexpr int LDK = DK, LDV = DV, LDC = kBC, NZ = NORM ? 16 : 0;
  static constexpr int QRL = kBC * LDK, QTL = DK * LDC, VRL = kBC * LDV, VTL = (DV + NZ) * LDC,
                       STL = (DV + NZ) * LDK, DNL = kBC * LDV, DTL = (DV + NZ) * LDC;
  static constexpr int QT = 0;                                // phi(Q)^T [dk][token]
  static constexpr int KT = QT + 2 * QTL;                     // phi(K)^T [dk][token]
  static constexpr int VR = KT + 2 * QTL;                     // V [token][dv]
  static constexpr int VT = VR + (VLO ? 2 : 1) * VRL;         // V^T [dv + 16 ones][token]; lo: dv rows
  static constexpr int ST = VT + VTL + (VLO ? DV * LDC : 0);  // S^T [dv + 16 z][dk]
  // the rows of phi(Q) and phi(K) are last read by the scores, and dnum takes
  // their place after a barrier
  static constexpr int U = ST + 2 * STL;
  static constexpr int QR = U;                                // phi(Q) [token][dk]
  static constexpr int KR = QR + 2 * QRL;                     // phi(K) [token][dk]
  static constexpr int DN = U;                                // dnum [token][dv]
  static constexpr int DT = DN + 2 * DNL;                     // dnum^T [dv + 16 dden parts][token]
  static constexpr int TOTAL = U + (4 * QRL > 2 * DNL + 2 * DTL ? 4 * QRL : 2 * DNL + 2 * DTL);
};

template <typename IT, int DK, int DV, bool NORM>
__global__ __launch_bounds__(kBT, 4) void bwd_fwd_kernel(BwdChunkArgs a) {
  constexpr bool VLO = !std::is_same_v<IT, uint16_t>;  // fp16 values are not exact in bf16
  using Ly = FwdLds<DK, DV, NORM, VLO>;
  constexpr int LDK = Ly::LDK, LDV = Ly::LDV, LDC = Ly::LDC;
  constexpr int NET = DV / 16, NDT = DK / 16, NZT = NORM ? 1 : 0;
  constexpr int NST = NDT * (NET + NZT);  // 16x16 tiles of S (+ z) and of the dS sum
  constexpr int TPW = (NST + kBW - 1) / kBW;
  constexpr int KSK = DK / 32, KSV = DV / 32;
  constexpr int NIQ = (kBC / 2) * (DK / 8), NIV = (kBC / 2) * (DV / 8);
  static_assert(2 * NIQ + NIV <= kBT && NIQ % 64 == 0 && NIV % 64 == 0, "one staging item per thread");
  __shared__ __align__(16) uint16_t sm[Ly::TOTAL];
  __shared__ float part[NORM ? NET * kBC : 1];  // dden_i parts per value tile

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int l = tid & 63, lr = l & 15, lg = l >> 4;  // re-derived per phase (see refresh)
  const int u = blockIdx.x / a.nseg, s = blockIdx.x % a.nseg;
  const int T = a.T, H = a.H;
  const int b = u / H, h = u % H;
  const int t0 = s * a.seg_len;
  const int t1 = min(T, t0 + a.seg_len);
  const int64_t HDK = (int64_t)H * DK, HDV = (int64_t)H * DV;
  const IT* qb = (const IT*)a.q + (int64_t)b * T * HDK + (int64_t)h * DK;
  const IT* kb = (const IT*)a.k + (int64_t)b * T * HDK + (int64_t)h * DK;
  const IT* vb = (const IT*)a.v + (int64_t)b * T * HDV + (int64_t)h * DV;
  const IT* yb = (const IT*)a.dy + (int64_t)b * T * HDV + (int64_t)h * DV;
  IT* dqb = (IT*)a.dq + (int64_t)b * T * HDK + (int64_t)h * DK;
  float* rdb = NORM ? a.rden + (int64_t)b * T * H + h : nullptr;
  float* ddb = NORM ? a.dden + (int64_t)b * T * H + h : nullptr;
  const uint8_t* mb = a.mask ? a.mask + (int64_t)b * T : nullptr;
  const float eps = a.eps;
  const bool elu = a.fm == kEluPlusOne;

  // ---- S (+ z) tiles and the dS (+ dz) sum: wave w owns tiles w + 8k; tile
  // (dt, et) holds rows 16dt + 4lg + q (dk), column 16et + lr (dv); the z tile
  // (et = NET) holds z in every column (the ones rows of V^T), the dz tile the
  // parts of dden in columns 0 .. NET-1
  f32x4_t st[TPW], ds[TPW];
  auto tile = [&](int k, int& dt, int& et) {
    const int tau = w + kBW * k;
    dt = tau / (NET + NZT);
    et = tau % (NET + NZT);
    return tau < NST;
  };
  {
    StartState<DK, DV, NORM> ss(a, u, s, s);
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      int dt, et;
      const bool on = tile(k, dt, et);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d = 16 * dt + 4 * lg + q;
        st[k][q] = on ? ss.at(d, et < NET ? 16 * et + lr : -1) : 0.f;
        ds[k][q] = 0.f;
      }
    }
  }
  if constexpr (NORM) {
    // ones rows of V^T
    for (int i = tid; i < 16 * LDC; i += kBT) sm[Ly::VT + DV * LDC + i] = 0x3f80;  // bf16 1.0
  }

  // ---- the segment's buffers (token t at byte (t - t0) * row)
  constexpr uint32_t ESZ = sizeof(IT);
  const uint32_t nt = (uint32_t)(t1 - t0);
  const uint32_t RK = (uint32_t)HDK * ESZ, RV = (uint32_t)HDV * ESZ;  // row bytes
  const rsrc_t rq = make_rsrc(qb + t0 * HDK, (nt - 1) * RK + DK * ESZ);
  const rsrc_t rk = make_rsrc(kb + t0 * HDK, (nt - 1) * RK + DK * ESZ);
  const rsrc_t rv = make_rsrc(vb + t0 * HDV, (nt - 1) * RV + DV * ESZ);
  const rsrc_t ry = make_rsrc(yb + t0 * HDV, (nt - 1) * RV + DV * ESZ);
  const rsrc_t rdq = make_rsrc(dqb + t0 * HDK, (nt - 1) * RK + DK * ESZ);
  const rsrc_t rrd = make_rsrc(NORM ? rdb + (int64_t)t0 * H : (const float*)qb, NORM ? ((nt - 1) * H + 1) * 4 : 0);
  const rsrc_t rdd = make_rsrc(NORM ? ddb + (int64_t)t0 * H : (const float*)qb, NORM ? ((nt - 1) * H + 1) * 4 : 0);
  const rsrc_t rmk = make_rsrc(mb ? mb + t0 : (const uint8_t*)qb, mb ? nt : 0);  // (no mask: read as 0, ignored)

  // ---- prefetch registers: the next chunk's data, consumed before they are
  // loaded again and tested only where they are used (a loaded value tested
  // or copied early would make the wave wait for every load issued before it)
  const Item it = make_item<NIQ, DK / 8, NIQ, DK / 8, NIV, DV / 8>(tid);
  const int im = it.on ? it.m : 0;  // (threads without an item read block 0 of q)
  const rsrc_t ir = im == 0 ? rq : (im == 1 ? rk : rv);
  const uint32_t irow = im == 2 ? RV : RK;
  u32x4_t raw[2];
  uint32_t rm0 = 1, rm1 = 1;         // mask bytes of the item's tokens
  int iq = 16 * (w & 1) + lr;  // query row of the lane in a chunk (phases B, C)
  u32x2_t dyraw = u32x2_t{0u, 0u};   // dy of the lane's query at value dims 16(w >> 1) + 4lg .. +3 (phase B)
  u32x2_t qraw = u32x2_t{0u, 0u};    // q of the lane's query at key dims 16(w >> 1) + 4lg .. +3 (phase C)
  uint32_t qm = 1;                   // mask byte of the lane's query
  const uint32_t ycol = (16 * min(w >> 1, NET - 1) + 4 * lg) * ESZ, qcol = (16 * min(w >> 1, NDT - 1) + 4 * lg) * ESZ;
  auto prefetch_items = [&](int c0) {
    const uint32_t ta = (uint32_t)(c0 - t0 + 2 * it.p);
    raw[0] = bload16(ir, ta * irow + 16 * it.cb);
    raw[1] = bload16(ir, (ta + 1) * irow + 16 * it.cb);
    rm0 = bload1(rmk, ta);
    rm1 = bload1(rmk, ta + 1);
  };
  auto prefetch_lane = [&](int c0) {
    const uint32_t t = (uint32_t)(c0 - t0 + iq);
    qm = bload1(rmk, t);
    dyraw = bload8(ry, t * RV + ycol);
    qraw = bload8(rq, t * RK + qcol);
  };
  // the item's token 2p + n of the chunk at c0 exists and is not masked
  auto item_ok = [&](int c0, int n) { return c0 + 2 * it.p + n < t1 && (mb == nullptr || (n ? rm1 : rm0) != 0u); };

  // ---- staging of phi(Q), phi(K), V (rows and transposed) and of S
  auto stage = [&](int c0) {
    if (!it.on) return;
    const bool ok0 = item_ok(c0, 0), ok1 = item_ok(c0, 1);
    u32x4_t h[2], lo[2];
    if (!VLO && im == 2) {
      // bf16 values are exact: the loaded words, no lo part
      const u32x4_t z4 = u32x4_t{0u, 0u, 0u, 0u};
      h[0] = ok0 ? raw[0] : z4;
      h[1] = ok1 ? raw[1] : z4;
    } else {
      float f[2][8];
      Io<IT>::unpack(raw[0], f[0]);
      Io<IT>::unpack(raw[1], f[1]);
      if (im == 2)
        split_rows<kEluPlusOne, false>(f, ok0, ok1, eps, h, lo);
      else if (elu)
        split_rows<kEluPlusOne, true>(f, ok0, ok1, eps, h, lo);
      else
        split_rows<kReluEps, true>(f, ok0, ok1, eps, h, lo);
    }
    const int rbase = im == 0 ? Ly::QR : (im == 1 ? Ly::KR : Ly::VR);
    const int rlo = im == 2 ? Ly::VRL : Ly::QRL;
    const int tbase = im == 0 ? Ly::QT : (im == 1 ? Ly::KT : Ly::VT);
    const int tlo = im == 2 ? Ly::VTL : Ly::QTL;
    const bool lo_too = im < 2 || VLO;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int off = rbase + (im == 2 ? ro<DV>(2 * it.p + n, 8 * it.cb) : ro<DK>(2 * it.p + n, 8 * it.cb));
      st16(sm + off, h[n]);
      if (lo_too) st16(sm + off + rlo, lo[n]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int off = tbase + to(8 * it.cb + e, 2 * it.p);
      *(uint32_t*)(sm + off) = tword(h[0], h[1], e);
      if (lo_too) *(uint32_t*)(sm + off + tlo) = tword(lo[0], lo[1], e);
    }
  };
  auto write_s = [&]() {
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      int dt, et;
      if (!tile(k, dt, et)) continue;
      u32x2_t hw, lw;
      { const u32x2_t t2_ = split2(st[k][0], st[k][1]); hw[0] = t2_[0]; lw[0] = t2_[1]; }
      { const u32x2_t t2_ = split2(st[k][2], st[k][3]); hw[1] = t2_[0]; lw[1] = t2_[1]; }
      const int off = Ly::ST + ro<DK>(et < NET ? 16 * et + lr : DV + lr, 16 * dt + 4 * lg);
      *(u32x2_t*)(sm + off) = hw;
      *(u32x2_t*)(sm + off + Ly::STL) = lw;
    }
  };

  const int nch = (t1 - t0 + kBC - 1) / kBC;
  if (nch > 0) {
    prefetch_items(t0);
    prefetch_lane(t0);
  }
  // lane indices re-derived in every phase: the addresses formed from them are
  // then computed where used instead of hoisted out of the loop and spilled
  auto refresh = [&]() {
    l = opaque_lane(tid);
    lr = l & 15;
    lg = l >> 4;
    iq = 16 * (w & 1) + lr;
  };
  for (int c = 0; c < nch; ++c) {
    const int cb0 = t0 + c * kBC;
    refresh();
    stage(cb0);
    write_s();
    const bool qvc = cb0 + iq < t1 && (mb == nullptr || qm != 0u);
    if (c + 1 < nch) prefetch_items(cb0 + kBC);
    __syncthreads();

    // ---- phase B: num, den of the wave's query block (w & 1) and value tile
    // (w >> 1); dnum, and the wave's part of dden
    refresh();
    u32x4_t ph, pl;
    // num^T, den^T tiles: rows 16et + 4lg + q (dv), column iq; their state
    // terms are formed with the phi(Q) rows before those are overwritten
    f32x4_t nacc = f32x4_t{0.f, 0.f, 0.f, 0.f}, dacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (w < 2 * NET) {
      const int et = w >> 1;
      u32x4_t qh[KSK], ql[KSK];
#pragma unroll
      for (int ks = 0; ks < KSK; ++ks) {
        qh[ks] = ld16(sm + Ly::QR + ro<DK>(iq, 32 * ks + 8 * lg));
        ql[ks] = ld16(sm + Ly::QR + Ly::QRL + ro<DK>(iq, 32 * ks + 8 * lg));
      }
      // scores P_ij = phi_q_i . phi_k_j, j <= i: lane holds keys 8lg..8lg+7 of query iq
      {
        f32x4_t at[2];
#pragma unroll
        for (int odd = 0; odd < 2; ++odd) {
          const int krow = 8 * (lr >> 2) + 4 * odd + (lr & 3);
          at[odd] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KSK; ++ks) {
            const int o = Ly::KR + ro<DK>(krow, 32 * ks + 8 * lg);
            mm3(at[odd], ld16(sm + o), ld16(sm + o + Ly::QRL), qh[ks], ql[ks]);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) at[odd][q] = (8 * lg + 4 * odd + q <= iq) ? at[odd][q] : 0.f;
        }
        pair_operand(at, ph, pl);
      }
#pragma unroll
      for (int ks = 0; ks < KSK; ++ks) {
        const int so = Ly::ST + ro<DK>(16 * et + lr, 32 * ks + 8 * lg);
        mm3(nacc, ld16(sm + so), ld16(sm + so + Ly::STL), qh[ks], ql[ks]);
      }
      if constexpr (NORM) {
#pragma unroll
        for (int ks = 0; ks < KSK; ++ks) {
          const int so = Ly::ST + ro<DK>(DV + lr, 32 * ks + 8 * lg);
          mm3(dacc, ld16(sm + so), ld16(sm + so + Ly::STL), qh[ks], ql[ks]);
        }
      }
    }
    __syncthreads();  // the phi(Q), phi(K) rows are read: dnum goes in their place
    refresh();
    if constexpr (NORM) {
      // the unused dden rows of dnum^T (the staging of phi(K) rows wrote there)
      for (int i = tid; i < (16 - NET) * LDC; i += kBT) {
        sm[Ly::DT + (DV + NET) * LDC + i] = 0;
        sm[Ly::DT + Ly::DTL + (DV + NET) * LDC + i] = 0;
      }
    }
    if (w < 2 * NET) {
      const int et = w >> 1;
      {
        const int o = Ly::VT + to(16 * et + lr, 8 * lg);
        const u32x4_t vh = ld16(sm + o);
        mm(nacc, vh, ph);
        mm(nacc, vh, pl);
        if constexpr (VLO) mm(nacc, ld16(sm + o + Ly::VTL), ph);
      }
      float rden = 1.f;
      if constexpr (NORM) {
        const u32x4_t vh = ld16(sm + Ly::VT + to(DV + lr, 8 * lg));
        mm(dacc, vh, ph);
        mm(dacc, vh, pl);
        rden = 1.f / (dacc[0] + eps);
      }
      f32x4_t dn;
#pragma unroll
      for (int q = 0; q < 4; ++q) dn[q] = qvc ? io_at<IT>(dyraw[q >> 1], q & 1) * rden : 0.f;
      // dnum rows (dv contiguous) and dnum^T (token contiguous)
      u32x2_t hw, lw;
      { const u32x2_t t2_ = split2(dn[0], dn[1]); hw[0] = t2_[0]; lw[0] = t2_[1]; }
      { const u32x2_t t2_ = split2(dn[2], dn[3]); hw[1] = t2_[0]; lw[1] = t2_[1]; }
      {
        const int o = Ly::DN + ro<DV>(iq, 16 * et + 4 * lg);
        *(u32x2_t*)(sm + o) = hw;
        *(u32x2_t*)(sm + o + Ly::DNL) = lw;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int o = Ly::DT + to(16 * et + 4 * lg + q, iq);
        sm[o] = (uint16_t)(q & 1 ? hw[q >> 1] >> 16 : hw[q >> 1] & 0xffffu);
        sm[o + Ly::DTL] = (uint16_t)(q & 1 ? lw[q >> 1] >> 16 : lw[q >> 1] & 0xffffu);
      }
      if constexpr (NORM) {
        float p = dn[0] * nacc[0] + dn[1] * nacc[1] + dn[2] * nacc[2] + dn[3] * nacc[3];
        p += __shfl_xor(p, 16);
        p += __shfl_xor(p, 32);
        const float pd = -p * rden;
        if (lg == 0) {
          part[et * kBC + iq] = pd;
          uint32_t ph1, pl1;
          split1(pd, ph1, pl1);
          sm[Ly::DT + to(DV + et, iq)] = (uint16_t)ph1;
          sm[Ly::DT + Ly::DTL + to(DV + et, iq)] = (uint16_t)pl1;
        }
      }
      if constexpr (NORM)
        bstore4(rrd, (et == 0 && lg == 0) ? (uint32_t)(cb0 - t0 + iq) * (uint32_t)H * 4 : kDrop,
                __float_as_uint(qvc ? rden : 0.f));
    }
    __syncthreads();

    // ---- phase C: dq of the wave's query block (w & 1) and key-dim tile (w >> 1)
    refresh();
    if (w < 2 * NDT) {
      const int dt = w >> 1;
      const uint32_t tr = (uint32_t)(cb0 - t0 + iq);  // the query's row in the segment
      float dd = 0.f;
      if constexpr (NORM) {
#pragma unroll
        for (int et = 0; et < NET; ++et) dd += part[et * kBC + iq];
        bstore4(rdd, (dt == 0 && lg == 0) ? tr * (uint32_t)H * 4 : kDrop, __float_as_uint(dd));
      }
      u32x4_t dh[KSV], dl[KSV];
#pragma unroll
      for (int ks = 0; ks < KSV; ++ks) {
        dh[ks] = ld16(sm + Ly::DN + ro<DV>(iq, 32 * ks + 8 * lg));
        dl[ks] = ld16(sm + Ly::DN + Ly::DNL + ro<DV>(iq, 32 * ks + 8 * lg));
      }
      // B_ij = dnum_i . v_j + dden_i, j <= i: keys 8lg..8lg+7 of query iq
      u32x4_t bh, bl;
      {
        f32x4_t at[2];
#pragma unroll
        for (int odd = 0; odd < 2; ++odd) {
          const int krow = 8 * (lr >> 2) + 4 * odd + (lr & 3);
          at[odd] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KSV; ++ks) {
            const int o = Ly::VR + ro<DV>(krow, 32 * ks + 8 * lg);
            const u32x4_t vh = ld16(sm + o);
            mm(at[odd], vh, dh[ks]);
            mm(at[odd], vh, dl[ks]);
            if constexpr (VLO) mm(at[odd], ld16(sm + o + Ly::VRL), dh[ks]);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) at[odd][q] = (8 * lg + 4 * odd + q <= iq) ? at[odd][q] + dd : 0.f;
        }
        pair_operand(at, bh, bl);
      }
      // dphi_q^T tile: rows 16dt + 4lg + q (dk), column iq
      f32x4_t g = f32x4_t{0.f, 0.f, 0.f, 0.f};
      {
        const int o = Ly::KT + to(16 * dt + lr, 8 * lg);
        mm3(g, ld16(sm + o), ld16(sm + o + Ly::QTL), bh, bl);
#pragma unroll
        for (int ks = 0; ks < KSV; ++ks) {
          // S rows (dv contiguous) gathered from S^T
          mm3(g, gather8<DK>(sm + Ly::ST, 32 * ks + 8 * lg, 16 * dt + lr),
              gather8<DK>(sm + Ly::ST + Ly::STL, 32 * ks + 8 * lg, 16 * dt + lr), dh[ks], dl[ks]);
        }
      }
      if constexpr (NORM) {
        const int zo = Ly::ST + ro<DK>(DV, 16 * dt + 4 * lg);
        const u32x2_t zh = *(const u32x2_t*)(sm + zo), zl = *(const u32x2_t*)(sm + zo + Ly::STL);
#pragma unroll
        for (int q = 0; q < 4; ++q) g[q] += (bf_at(zh[q >> 1], q & 1) + bf_at(zl[q >> 1], q & 1)) * dd;
      }
      {
        float o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = qvc ? g[q] * dphi_rt(io_at<IT>(qraw[q >> 1], q & 1), elu) : 0.f;
        bstore8(rdq, tr * RK + (16 * dt + 4 * lg) * ESZ, pack4<IT>(o[0], o[1], o[2], o[3]));
      }
    }

    // dy, q and the mask byte of the lane's next query (this chunk's are used)
    if (c + 1 < nch) prefetch_lane(cb0 + kBC);

    // ---- phase D: S += phiK^T V (z += phiK^T 1), dS += phiQ^T dnum (dz parts += phiQ^T dden parts)
    refresh();
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      int dt, et;
      if (!tile(k, dt, et)) continue;
      const int ao = to(16 * dt + lr, 8 * lg);
      const int bo = to(et < NET ? 16 * et + lr : DV + lr, 8 * lg);
      const u32x4_t kh = ld16(sm + Ly::KT + ao), kl = ld16(sm + Ly::KT + Ly::QTL + ao);
      const u32x4_t vh = ld16(sm + Ly::VT + bo);
      mm(st[k], kh, vh);
      mm(st[k], kl, vh);
      if constexpr (VLO) {
        if (et < NET) mm(st[k], kh, ld16(sm + Ly::VT + Ly::VTL + bo));
      }
      mm3(ds[k], ld16(sm + Ly::QT + ao), ld16(sm + Ly::QT + Ly::QTL + ao), ld16(sm + Ly::DT + bo),
          ld16(sm + Ly::DT + Ly::DTL + bo));
    }
    __syncthreads();
  }

  // ---- the segment's dS (dz) sum -> slot nseg - s for the reverse prefix
  if (s >= 1) {
    const int r = a.nseg - s;
    float* so = a.s_out + u * a.s_out_u + r * a.s_out_s;
    float* zo = (NORM && a.z_out) ? a.z_out + u * a.z_out_u + r * a.z_out_s : nullptr;
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      int dt, et;
      if (!tile(k, dt, et)) continue;
      if (et < NET) {
#pragma unroll
        for (int q = 0; q < 4; ++q) so[(16 * dt + 4 * lg + q) * DV + 16 * et + lr] = ds[k][q];
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float z = 0.f;
#pragma unroll
          for (int c2 = 0; c2 < NET; ++c2) z += __shfl(ds[k][q], 16 * lg + c2);
          if (lr == 0 && zo) zo[16 * dt + 4 * lg + q] = z;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Segment sums of the forward state, sum phi_k v^T (and sum phi_k), in the
// same hi + lo precision: the state at a segment start enters the gradients
// through the same cancelling terms.  Workgroup blockIdx sums segment
// s = blockIdx % nseg of unit blockIdx / nseg into slot s + 1, in 64-token
// chunks (twice the forward passes' 32: half the chain of loads and barriers).
constexpr int kSC = 64;
template <int DK, int DV, bool NORM, bool VLO>
struct StateLds {
  static constexpr int LDC = kSC, NZ = NORM ? 16 : 0;  // rows of kSC tokens, swizzled as row tiles
  static constexpr int KTL = DK * LDC, VTL = (DV + NZ) * LDC;
  static constexpr int KT = 0;              // phi(K)^T [dk][token], hi then lo
  static constexpr int VT = KT + 2 * KTL;   // V^T [dv + 16 ones][token]; lo: dv rows
  static constexpr int TOTAL = VT + VTL + (VLO ? DV * LDC : 0);
};

template <typename IT, int DK, int DV, bool NORM>
__global__ __launch_bounds__(kBT, 2) void bwd_state_kernel(BwdChunkArgs a) {
  constexpr bool VLO = !std::is_same_v<IT, uint16_t>;
  using Ly = StateLds<DK, DV, NORM, VLO>;
  constexpr int LDC = Ly::LDC;
  constexpr int NET = DV / 16, NDT = DK / 16, NZT = NORM ? 1 : 0;
  constexpr int NST = NDT * (NET + NZT);
  constexpr int TPW = (NST + kBW - 1) / kBW;
  constexpr int NIK = (kSC / 2) * (DK / 8), NIV = (kSC / 2) * (DV / 8);
  static_assert(NIK + NIV <= kBT && NIK % 64 == 0 && NIV % 64 == 0, "one staging item per thread");
  __shared__ __align__(16) uint16_t sm[Ly::TOTAL];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, lr = l & 15, lg = l >> 4;
  const int u = blockIdx.x / a.nseg, s = blockIdx.x % a.nseg;
  const int T = a.T, H = a.H;
  const int b = u / H, h = u % H;
  const int t0 = s * a.seg_len;
  const int t1 = min(T, t0 + a.seg_len);
  const int64_t HDK = (int64_t)H * DK, HDV = (int64_t)H * DV;
  const IT* kb = (const IT*)a.k + (int64_t)b * T * HDK + (int64_t)h * DK;
  const IT* vb = (const IT*)a.v + (int64_t)b * T * HDV + (int64_t)h * DV;
  const uint8_t* mb = a.mask ? a.mask + (int64_t)b * T : nullptr;
  const float eps = a.eps;
  const bool elu = a.fm == kEluPlusOne;

  f32x4_t st[TPW];
  auto tile = [&](int k, int& dt, int& et) {
    const int tau = w + kBW * k;
    dt = tau / (NET + NZT);
    et = tau % (NET + NZT);
    return tau < NST;
  };
#pragma unroll
  for (int k = 0; k < TPW; ++k) st[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (NORM) {
    for (int i = tid; i < 16 * LDC; i += kBT) sm[Ly::VT + DV * LDC + i] = 0x3f80;  // bf16 1.0
  }

  constexpr uint32_t ESZ = sizeof(IT);
  const uint32_t nt = (uint32_t)(t1 - t0);
  const uint32_t RK = (uint32_t)HDK * ESZ, RV = (uint32_t)HDV * ESZ;
  const rsrc_t rk = make_rsrc(kb + t0 * HDK, (nt - 1) * RK + DK * ESZ);
  const rsrc_t rv = make_rsrc(vb + t0 * HDV, (nt - 1) * RV + DV * ESZ);
  const rsrc_t rmk = make_rsrc(mb ? mb + t0 : (const uint8_t*)kb, mb ? nt : 0);
  const Item it = make_item<NIK, DK / 8, NIV, DV / 8, 0, 1>(tid);  // m: 0 k, 1 v
  const int im = it.on ? it.m : 0;  // (threads without an item read block 0 of k)
  const rsrc_t ir = im == 0 ? rk : rv;
  const uint32_t irow = im == 0 ? RK : RV;
  // (buffer loads, mask bytes tested at the stage: see the forward pass)
  u32x4_t raw0, raw1;
  uint32_t rm0 = 1, rm1 = 1;
  auto prefetch = [&](int c0) {
    const uint32_t ta = (uint32_t)(c0 - t0 + 2 * it.p);
    raw0 = bload16(ir, ta * irow + 16 * it.cb);
    raw1 = bload16(ir, (ta + 1) * irow + 16 * it.cb);
    rm0 = bload1(rmk, ta);
    rm1 = bload1(rmk, ta + 1);
  };
  auto stage = [&](int c0) {
    if (!it.on) return;
    const bool ok0 = c0 + 2 * it.p < t1 && (mb == nullptr || rm0 != 0u);
    const bool ok1 = c0 + 2 * it.p + 1 < t1 && (mb == nullptr || rm1 != 0u);
    u32x4_t h[2], lo[2];
    if (!VLO && im == 1) {
      const u32x4_t z4 = u32x4_t{0u, 0u, 0u, 0u};
      h[0] = ok0 ? raw0 : z4;
      h[1] = ok1 ? raw1 : z4;
    } else {
      float f[2][8];
      Io<IT>::unpack(raw0, f[0]);
      Io<IT>::unpack(raw1, f[1]);
      if (im == 1)
        split_rows<kEluPlusOne, false>(f, ok0, ok1, eps, h, lo);
      else if (elu)
        split_rows<kEluPlusOne, true>(f, ok0, ok1, eps, h, lo);
      else
        split_rows<kReluEps, true>(f, ok0, ok1, eps, h, lo);
    }
    const int tbase = im == 0 ? Ly::KT : Ly::VT;
    const int tlo = im == 0 ? Ly::KTL : Ly::VTL;
    const bool lo_too = im == 0 || VLO;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int off = tbase + ro<kSC>(8 * it.cb + e, 2 * it.p);
      *(uint32_t*)(sm + off) = tword(h[0], h[1], e);
      if (lo_too) *(uint32_t*)(sm + off + tlo) = tword(lo[0], lo[1], e);
    }
  };

  const int nch = (t1 - t0 + kSC - 1) / kSC;
  if (nch > 0) prefetch(t0);
  for (int c = 0; c < nch; ++c) {
    stage(t0 + c * kSC);
    if (c + 1 < nch) prefetch(t0 + (c + 1) * kSC);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      int dt, et;
      if (!tile(k, dt, et)) continue;
#pragma unroll
      for (int ks = 0; ks < kSC / 32; ++ks) {
        const int ao = Ly::KT + ro<kSC>(16 * dt + lr, 32 * ks + 8 * lg);
        const int bo = Ly::VT + ro<kSC>(et < NET ? 16 * et + lr : DV + lr, 32 * ks + 8 * lg);
        const u32x4_t kh = ld16(sm + ao), kl = ld16(sm + ao + Ly::KTL), vh = ld16(sm + bo);
        mm(st[k], kh, vh);
        mm(st[k], kl, vh);
        if constexpr (VLO) {
          if (et < NET) mm(st[k], kh, ld16(sm + bo + Ly::VTL));
        }
      }
    }
    __syncthreads();
  }

  float* so = a.s_out + u * a.s_out_u + (s + 1) * a.s_out_s;
  float* zo = (NORM && a.z_out) ? a.z_out + u * a.z_out_u + (s + 1) * a.z_out_s : nullptr;
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    int dt, et;
    if (!tile(k, dt, et)) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d = 16 * dt + 4 * lg + q;
      if (et < NET)
        so[d * DV + 16 * et + lr] = st[k][q];
      else if (zo && lr == 0)
        zo[d] = st[k][q];
    }
  }
}

// ---------------------------------------------------------------------------
// Reverse pass: LDS layout in 16-bit elements.
template <int DK, int DV, bool NORM, bool VLO>
struct RevLds {
  static constexpr int LDK = DK, LDV = DV, LDC = kBC, NZ = NORM ? 16 : 0;
  static constexpr int QRL = kBC * LDK, QTL = DK * LDC, VRL = kBC * LDV, DNL = kBC * LDV, DTL = (DV + NZ) * LDC,
                       SAL = DV * LDK;
  static constexpr int QR = 0;                         // phi(Q) [token][dk]
  static constexpr int QT = QR + 2 * QRL;              // phi(Q)^T [dk][token]
  static constexpr int KR = QT + 2 * QTL;              // phi(K) [token][dk]
  static constexpr int VR = KR + 2 * QRL;              // V [token][dv]
  static constexpr int DN = VR + (VLO ? 2 : 1) * VRL;  // dnum [token][dv]
  static constexpr int DT = DN + 2 * DNL;              // dnum^T [dv + 16: dden, zeros][token]
  static constexpr int SA = DT + 2 * DTL;              // dS^T [dv][dk]
  static constexpr int TOTAL = SA + 2 * SAL;
};

template <typename IT, int DK, int DV, bool NORM>
__global__ __launch_bounds__(kBT, 4) void bwd_rev_kernel(BwdChunkArgs a) {
  constexpr bool VLO = !std::is_same_v<IT, uint16_t>;
  using Ly = RevLds<DK, DV, NORM, VLO>;
  constexpr int LDK = Ly::LDK, LDV = Ly::LDV, LDC = Ly::LDC;
  constexpr int NET = DV / 16, NDT = DK / 16, NZT = NORM ? 1 : 0;
  constexpr int NST = NDT * (NET + NZT);
  constexpr int TPW = (NST + kBW - 1) / kBW;
  constexpr int KSK = DK / 32, KSV = DV / 32;
  constexpr int NIQ = (kBC / 2) * (DK / 8), NIV = (kBC / 2) * (DV / 8);
  static_assert(2 * NIQ + 2 * NIV <= kBT && NIQ % 64 == 0 && NIV % 64 == 0, "one staging item per thread");
  __shared__ __align__(16) uint16_t sm[Ly::TOTAL];
  __shared__ float dzv[NORM ? DK : 1], ddv[NORM ? kBC : 1];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int l = tid & 63, lr = l & 15, lg = l >> 4;  // re-derived per phase (see refresh)
  const int u = blockIdx.x / a.nseg, s = blockIdx.x % a.nseg;
  const int T = a.T, H = a.H;
  const int b = u / H, h = u % H;
  const int t0 = s * a.seg_len;
  const int t1 = min(T, t0 + a.seg_len);
  const int64_t HDK = (int64_t)H * DK, HDV = (int64_t)H * DV;
  const IT* qb = (const IT*)a.q + (int64_t)b * T * HDK + (int64_t)h * DK;
  const IT* kb = (const IT*)a.k + (int64_t)b * T * HDK + (int64_t)h * DK;
  const IT* vb = (const IT*)a.v + (int64_t)b * T * HDV + (int64_t)h * DV;
  const IT* yb = (const IT*)a.dy + (int64_t)b * T * HDV + (int64_t)h * DV;
  const float* rdb = NORM ? a.rden + (int64_t)b * T * H + h : nullptr;
  const float* ddb = NORM ? a.dden + (int64_t)b * T * H + h : nullptr;
  IT* dkb = (IT*)a.dk + (int64_t)b * T * HDK + (int64_t)h * DK;
  IT* dvb = (IT*)a.dv + (int64_t)b * T * HDV + (int64_t)h * DV;
  const uint8_t* mb = a.mask ? a.mask + (int64_t)b * T : nullptr;
  const float eps = a.eps;
  const bool elu = a.fm == kEluPlusOne;

  // ---- dS (+ dz) tiles: the gradient sums of the tokens after the current
  // chunk; the dz tile holds dz in column 0 (row DV of dnum^T is dden)
  f32x4_t ds[TPW];
  auto tile = [&](int k, int& dt, int& et) {
    const int tau = w + kBW * k;
    dt = tau / (NET + NZT);
    et = tau % (NET + NZT);
    return tau < NST;
  };
  {
    StartState<DK, DV, NORM> ss(a, u, a.nseg - 1 - s, a.nseg - 1 - s);
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      int dt, et;
      const bool on = tile(k, dt, et);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d = 16 * dt + 4 * lg + q;
        ds[k][q] = (on && (et < NET || lr == 0)) ? ss.at(d, et < NET ? 16 * et + lr : -1) : 0.f;
      }
    }
  }
  if constexpr (NORM) {
    for (int i = tid; i < 15 * LDC; i += kBT) {
      sm[Ly::DT + (DV + 1) * LDC + i] = 0;
      sm[Ly::DT + Ly::DTL + (DV + 1) * LDC + i] = 0;
    }
  }

  // ---- prefetch registers: q (rows and transposed), k (rows), v (rows), dy
  // (dnum rows and transposed, with 1/den of the item's two tokens)
  const Item it = make_item<NIQ, DK / 8, NIQ, DK / 8, NIV, DV / 8, NIV, DV / 8>(tid);
  // ---- the segment's buffers (token t at byte (t - t0) * row)
  constexpr uint32_t ESZ = sizeof(IT);
  const uint32_t nt = (uint32_t)(t1 - t0);
  const uint32_t RK = (uint32_t)HDK * ESZ, RV = (uint32_t)HDV * ESZ;
  const rsrc_t rq = make_rsrc(qb + t0 * HDK, (nt - 1) * RK + DK * ESZ);
  const rsrc_t rk = make_rsrc(kb + t0 * HDK, (nt - 1) * RK + DK * ESZ);
  const rsrc_t rv = make_rsrc(vb + t0 * HDV, (nt - 1) * RV + DV * ESZ);
  const rsrc_t ry = make_rsrc(yb + t0 * HDV, (nt - 1) * RV + DV * ESZ);
  const rsrc_t rrd = make_rsrc(NORM ? rdb + (int64_t)t0 * H : (const float*)qb, NORM ? ((nt - 1) * H + 1) * 4 : 0);
  const rsrc_t rdd = make_rsrc(NORM ? ddb + (int64_t)t0 * H : (const float*)qb, NORM ? ((nt - 1) * H + 1) * 4 : 0);
  const rsrc_t rdk = make_rsrc(dkb + t0 * HDK, (nt - 1) * RK + DK * ESZ);
  const rsrc_t rdv = make_rsrc(dvb + t0 * HDV, (nt - 1) * RV + DV * ESZ);
  const rsrc_t rmk = make_rsrc(mb ? mb + t0 : (const uint8_t*)qb, mb ? nt : 0);

  // ---- prefetch registers (buffer loads, tested where used: see the forward
  // pass).  The item's rows: a 16-byte block of q, k, v or dy (token 2p: raw0,
  // token 2p+1: raw2), and for dy the two tokens' 1/den (rd0, rd1).
  const int im = it.on ? it.m : 0;  // (threads without an item read block 0 of q)
  const bool idn = im == 3;
  const rsrc_t ir = im == 0 ? rq : (im == 1 ? rk : (im == 2 ? rv : ry));
  const uint32_t irow = im <= 1 ? RK : RV;
  const uint32_t iblk = 16 * it.cb;  // byte offset of the block in the row
  u32x4_t raw0, raw2;
  uint32_t rd0 = 0, rd1 = 0;
  uint32_t rm0 = 1, rm1 = 1;
  float ddn = 0.f;                   // dden of token tid % 32 of the chunk
  int jq = 16 * (w & 1) + lr;  // key row of the lane in a chunk (phases E, F)
  u32x2_t kraw = u32x2_t{0u, 0u};    // k of the lane's key at key dims 16(w >> 1) + 4lg .. +3 (phase F)
  uint32_t km = 1;                   // mask byte of the lane's key
  const uint32_t kcol = (16 * min(w >> 1, NDT - 1) + 4 * lg) * ESZ;
  auto prefetch_items = [&](int c0) {
    const uint32_t ta = (uint32_t)(c0 - t0 + 2 * it.p);
    raw0 = bload16(ir, ta * irow + iblk);
    raw2 = bload16(ir, (ta + 1) * irow + iblk);
    if constexpr (NORM) {
      rd0 = bload4(rrd, idn ? ta * (uint32_t)H * 4 : kDrop);
      rd1 = bload4(rrd, idn ? (ta + 1) * (uint32_t)H * 4 : kDrop);
    }
    rm0 = bload1(rmk, ta);
    rm1 = bload1(rmk, ta + 1);
    if constexpr (NORM) ddn = __uint_as_float(bload4(rdd, (uint32_t)(c0 - t0 + (tid & (kBC - 1))) * H * 4));
  };
  auto prefetch_lane = [&](int c0) {
    const uint32_t t = (uint32_t)(c0 - t0 + jq);
    km = bload1(rmk, t);
    kraw = bload8(rk, t * RK + kcol);
  };

  auto stage = [&](int c0) {
    if constexpr (NORM) {
      if (tid < kBC) {
        const float dd = c0 + tid < t1 ? ddn : 0.f;
        ddv[tid] = dd;
        uint32_t hh, ll;
        split1(dd, hh, ll);
        sm[Ly::DT + to(DV, tid)] = (uint16_t)hh;
        sm[Ly::DT + Ly::DTL + to(DV, tid)] = (uint16_t)ll;
      }
    }
    if (!it.on) return;
    const bool ok0 = c0 + 2 * it.p < t1 && (mb == nullptr || rm0 != 0u);
    const bool ok1 = c0 + 2 * it.p + 1 < t1 && (mb == nullptr || rm1 != 0u);
    u32x4_t h[2], lo[2];
    if (!VLO && im == 2) {
      const u32x4_t z4 = u32x4_t{0u, 0u, 0u, 0u};
      h[0] = ok0 ? raw0 : z4;
      h[1] = ok1 ? raw2 : z4;
    } else {
      float f[2][8];
      Io<IT>::unpack(raw0, f[0]);
      Io<IT>::unpack(raw2, f[1]);
      if (NORM && idn) {
        // dnum = dy / den, the forward pass's product
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          f[0][e] *= __uint_as_float(rd0);
          f[1][e] *= __uint_as_float(rd1);
        }
      }
      if (im >= 2)
        split_rows<kEluPlusOne, false>(f, ok0, ok1, eps, h, lo);
      else if (elu)
        split_rows<kEluPlusOne, true>(f, ok0, ok1, eps, h, lo);
      else
        split_rows<kReluEps, true>(f, ok0, ok1, eps, h, lo);
    }
    const int rbase = im == 0 ? Ly::QR : (im == 1 ? Ly::KR : (im == 2 ? Ly::VR : Ly::DN));
    const int rlo = im == 3 ? Ly::DNL : (im == 2 ? Ly::VRL : Ly::QRL);
    const bool lo_too = im != 2 || VLO;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int off = rbase + (im >= 2 ? ro<DV>(2 * it.p + n, 8 * it.cb) : ro<DK>(2 * it.p + n, 8 * it.cb));
      st16(sm + off, h[n]);
      if (lo_too) st16(sm + off + rlo, lo[n]);
    }
    if (im == 0 || im == 3) {
      // transposed: phi(Q)^T, dnum^T
      const int tbase = im == 0 ? Ly::QT : Ly::DT;
      const int tlo = im == 0 ? Ly::QTL : Ly::DTL;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int off = tbase + to(8 * it.cb + e, 2 * it.p);
        *(uint32_t*)(sm + off) = tword(h[0], h[1], e);
        *(uint32_t*)(sm + off + tlo) = tword(lo[0], lo[1], e);
      }
    }
  };
  auto write_ds = [&]() {
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      int dt, et;
      if (!tile(k, dt, et)) continue;
      if (et < NET) {
        u32x2_t hw, lw;
        { const u32x2_t t2_ = split2(ds[k][0], ds[k][1]); hw[0] = t2_[0]; lw[0] = t2_[1]; }
        { const u32x2_t t2_ = split2(ds[k][2], ds[k][3]); hw[1] = t2_[0]; lw[1] = t2_[1]; }
        const int off = Ly::SA + ro<DK>(16 * et + lr, 16 * dt + 4 * lg);
        *(u32x2_t*)(sm + off) = hw;
        *(u32x2_t*)(sm + off + Ly::SAL) = lw;
      } else if constexpr (NORM) {
        if (lr == 0) {
#pragma unroll
          for (int q = 0; q < 4; ++q) dzv[16 * dt + 4 * lg + q] = ds[k][q];
        }
      }
    }
  };

  const int nch = (t1 - t0 + kBC - 1) / kBC;
  if (nch > 0) {
    prefetch_items(t0 + (nch - 1) * kBC);
    prefetch_lane(t0 + (nch - 1) * kBC);
  }
  auto refresh = [&]() {
    l = opaque_lane(tid);
    lr = l & 15;
    lg = l >> 4;
    jq = 16 * (w & 1) + lr;
  };
  for (int c = nch - 1; c >= 0; --c) {
    refresh();
    const int cb0 = t0 + c * kBC;
    stage(cb0);
    write_ds();
    const int tj = cb0 + jq;
    const bool kvc = tj < t1 && (mb == nullptr || km != 0u);
    if (c > 0) prefetch_items(cb0 - kBC);
    __syncthreads();

    // ---- phase E: dv of the wave's key block (w & 1) and value tile (w >> 1)
    refresh();
    if (w < 2 * NET) {
      const int et = w >> 1;
      u32x4_t kh[KSK], kl[KSK];
#pragma unroll
      for (int ks = 0; ks < KSK; ++ks) {
        kh[ks] = ld16(sm + Ly::KR + ro<DK>(jq, 32 * ks + 8 * lg));
        kl[ks] = ld16(sm + Ly::KR + Ly::QRL + ro<DK>(jq, 32 * ks + 8 * lg));
      }
      // P_ij, i >= j: lane holds queries 8lg..8lg+7 of key jq
      u32x4_t ph, pl;
      {
        f32x4_t at[2];
#pragma unroll
        for (int odd = 0; odd < 2; ++odd) {
          const int qrow = 8 * (lr >> 2) + 4 * odd + (lr & 3);
          at[odd] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KSK; ++ks) {
            const int o = Ly::QR + ro<DK>(qrow, 32 * ks + 8 * lg);
            mm3(at[odd], ld16(sm + o), ld16(sm + o + Ly::QRL), kh[ks], kl[ks]);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) at[odd][q] = (8 * lg + 4 * odd + q >= jq) ? at[odd][q] : 0.f;
        }
        pair_operand(at, ph, pl);
      }
      // dv^T tile: rows 16et + 4lg + q (dv), column jq
      f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
      {
        const int o = Ly::DT + to(16 * et + lr, 8 * lg);
        mm3(acc, ld16(sm + o), ld16(sm + o + Ly::DTL), ph, pl);
#pragma unroll
        for (int ks = 0; ks < KSK; ++ks) {
          const int so = Ly::SA + ro<DK>(16 * et + lr, 32 * ks + 8 * lg);
          mm3(acc, ld16(sm + so), ld16(sm + so + Ly::SAL), kh[ks], kl[ks]);
        }
      }
      bstore8(rdv, (uint32_t)(tj - t0) * RV + (16 * et + 4 * lg) * ESZ,
              pack4<IT>(kvc ? acc[0] : 0.f, kvc ? acc[1] : 0.f, kvc ? acc[2] : 0.f, kvc ? acc[3] : 0.f));
    }

    // ---- phase F: dk of the wave's key block (w & 1) and key-dim tile (w >> 1)
    refresh();
    if (w < 2 * NDT) {
      const int dt = w >> 1;
      u32x4_t vh[KSV], vl[VLO ? KSV : 1];
#pragma unroll
      for (int ks = 0; ks < KSV; ++ks) {
        vh[ks] = ld16(sm + Ly::VR + ro<DV>(jq, 32 * ks + 8 * lg));
        if constexpr (VLO) vl[ks] = ld16(sm + Ly::VR + Ly::VRL + ro<DV>(jq, 32 * ks + 8 * lg));
      }
      // B_ij = dnum_i . v_j + dden_i, i >= j: queries 8lg..8lg+7 of key jq
      u32x4_t bh, bl;
      {
        f32x4_t at[2];
#pragma unroll
        for (int odd = 0; odd < 2; ++odd) {
          const int qrow = 8 * (lr >> 2) + 4 * odd + (lr & 3);
          at[odd] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KSV; ++ks) {
            const int o = Ly::DN + ro<DV>(qrow, 32 * ks + 8 * lg);
            const u32x4_t dh = ld16(sm + o), dl = ld16(sm + o + Ly::DNL);
            mm(at[odd], dh, vh[ks]);
            mm(at[odd], dl, vh[ks]);
            if constexpr (VLO) mm(at[odd], dh, vl[ks]);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int i = 8 * lg + 4 * odd + q;
            const float dd = NORM ? ddv[i] : 0.f;
            at[odd][q] = i >= jq ? at[odd][q] + dd : 0.f;
          }
        }
        pair_operand(at, bh, bl);
      }
      // dphi_k^T tile: rows 16dt + 4lg + q (dk), column jq
      f32x4_t g = f32x4_t{0.f, 0.f, 0.f, 0.f};
      {
        const int o = Ly::QT + to(16 * dt + lr, 8 * lg);
        mm3(g, ld16(sm + o), ld16(sm + o + Ly::QTL), bh, bl);
#pragma unroll
        for (int ks = 0; ks < KSV; ++ks) {
          // dS rows (dv contiguous) gathered from dS^T
          const u32x4_t sh = gather8<DK>(sm + Ly::SA, 32 * ks + 8 * lg, 16 * dt + lr),
                        sl = gather8<DK>(sm + Ly::SA + Ly::SAL, 32 * ks + 8 * lg, 16 * dt + lr);
          mm(g, sh, vh[ks]);
          mm(g, sl, vh[ks]);
          if constexpr (VLO) mm(g, sh, vl[ks]);
        }
      }
      if constexpr (NORM) {
#pragma unroll
        for (int q = 0; q < 4; ++q) g[q] += dzv[16 * dt + 4 * lg + q];
      }
      {
        float o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = kvc ? g[q] * dphi_rt(io_at<IT>(kraw[q >> 1], q & 1), elu) : 0.f;
        bstore8(rdk, (uint32_t)(tj - t0) * RK + (16 * dt + 4 * lg) * ESZ, pack4<IT>(o[0], o[1], o[2], o[3]));
      }
    }

    // k and the mask byte of the lane's key in the previous chunk (this chunk's are used)
    if (c > 0) prefetch_lane(cb0 - kBC);

    // ---- phase G: dS += phiQ^T dnum, dz += phiQ^T dden (column 0 of the dz tile)
    refresh();
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      int dt, et;
      if (!tile(k, dt, et)) continue;
      const int ao = to(16 * dt + lr, 8 * lg);
      const int bo = to(et < NET ? 16 * et + lr : DV + lr, 8 * lg);
      mm3(ds[k], ld16(sm + Ly::QT + ao), ld16(sm + Ly::QT + Ly::QTL + ao), ld16(sm + Ly::DT + bo),
          ld16(sm + Ly::DT + Ly::DTL + bo));
    }
    __syncthreads();
  }

  // ---- the first segment ends with dS_0, dz_0
  if (s == 0) {
    float* so = a.s_out + u * a.s_out_u;
    float* zo = (NORM && a.z_out) ? a.z_out + u * a.z_out_u : nullptr;
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      int dt, et;
      if (!tile(k, dt, et)) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d = 16 * dt + 4 * lg + q;
        if (et < NET)
          so[d * DV + 16 * et + lr] = ds[k][q];
        else if (zo && lr == 0)
          zo[d] = ds[k][q];
      }
    }
  }
}

template <typename IT, int DK, int DV, bool NORM>
hipError_t launch_bwd_chunk_t(int pass, const BwdChunkArgs& a, int grid, hipStream_t st) {
  if (pass == 0)
    hipLaunchKernelGGL((bwd_fwd_kernel<IT, DK, DV, NORM>), dim3(grid), dim3(kBT), 0, st, a);
  else if (pass == 1)
    hipLaunchKernelGGL((bwd_rev_kernel<IT, DK, DV, NORM>), dim3(grid), dim3(kBT), 0, st, a);
  else
    hipLaunchKernelGGL((bwd_state_kernel<IT, DK, DV, NORM>), dim3(grid), dim3(kBT), 0, st, a);
  return hipGetLastError();
}

template <typename IT, int DK, int DV>
hipError_t launch_bwd_chunk_n(int pass, int norm, const BwdChunkArgs& a, int grid, hipStream_t st) {
  return norm ? launch_bwd_chunk_t<IT, DK, DV, true>(pass, a, grid, st)
              : launch_bwd_chunk_t<IT, DK, DV, false>(pass, a, grid, st);
}

template <typename IT>
hipError_t launch_bwd_chunk_d(int pass, int Dk, int Dv, int norm, const BwdChunkArgs& a, int grid,
                              hipStream_t st) {
  if (Dk == 32 && Dv == 32) return launch_bwd_chunk_n<IT, 32, 32>(pass, norm, a, grid, st);
  if (Dk == 32 && Dv == 64) return launch_bwd_chunk_n<IT, 32, 64>(pass, norm, a, grid, st);
  if (Dk == 64 && Dv == 32) return launch_bwd_chunk_n<IT, 64, 32>(pass, norm, a, grid, st);
  if (Dk == 64 && Dv == 64) return launch_bwd_chunk_n<IT, 64, 64>(pass, norm, a, grid, st);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_bwd_chunk(int pass, int io, int Dk, int Dv, int norm, const BwdChunkArgs& a, int grid,
                            hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  if (io == kIoBF16) return launch_bwd_chunk_d<uint16_t>(pass, Dk, Dv, norm, a, grid, st);
  if (io == kIoF16) return launch_bwd_chunk_d<f16_t>(pass, Dk, Dv, norm, a, grid, st);
  return hipErrorInvalidValue;
}

}  // namespace la
