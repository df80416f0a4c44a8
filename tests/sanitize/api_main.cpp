// Drives the host side of liblinattn's C ABI (la_api.cpp: argument checks,
// planning, workspace sizing, dispatch) for a build with AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_sanitizers.py).  The kernel launchers
// are replaced by stubs that check their arguments and count launches, so no
// device is needed; the pointers are fake and never dereferenced.
#include <stdint.h>
#include <stdio.h>

#include "liblinattn.h"
#include "la_launch.hpp"

static int launches = 0, bad = 0;
static void seen(bool ok, const char* what) {
  ++launches;
  if (!ok) {
    ++bad;
    printf("bad launch arguments: %s\n", what);
  }
}

namespace la {
hipError_t launch_chunk(int mode, int io, int D, int fm, int norm, const ChunkArgs& a, int grid, hipStream_t) {
  seen(grid > 0 && a.T > 0 && a.H > 0 && a.seg_count > 0 && (mode == 0 || mode == 1) && io >= 0 && io <= 2 &&
           D >= 32 && fm >= 0 && norm >= 0,
       "chunk");
  return hipSuccess;
}
hipError_t launch_seg_prefix(float* s, float*, const float*, const float*, int U, int nseg, int dk, int dv, int,
                             hipStream_t) {
  seen(s && U > 0 && nseg > 1 && dk > 0 && dv > 0, "seg_prefix");
  return hipSuccess;
}
hipError_t launch_seg_sum(float* s, float*, int U, int nseg, int dk, int dv, int, hipStream_t) {
  seen(s && U > 0 && nseg > 0 && dk > 0 && dv > 0, "seg_sum");
  return hipSuccess;
}
int apply_groups_per_unit(int64_t U, int64_t T) { return T > 4096 ? 8 : (U > 0 ? 1 : 0); }
hipError_t launch_apply(int, int D, int, int, const ApplyArgs& a, int grid, hipStream_t) {
  seen(grid > 0 && a.s && D > 0, "apply");
  return hipSuccess;
}
hipError_t launch_decode(int, int Dk, int Dv, int, int, const DecodeArgs& a, int units, hipStream_t) {
  seen(units > 0 && a.s_in && a.s_out && Dk > 0 && Dv > 0, "decode");
  return hipSuccess;
}
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t) {
  seen(p && n > 0, "fill_zero");
  return hipSuccess;
}
hipError_t launch_copy(float* d, const float* s, int64_t n, hipStream_t) {
  seen(d && s && n > 0, "copy");
  return hipSuccess;
}
hipError_t launch_gated(int, int, int D, int G, const GatedArgs& a, int grid, hipStream_t) {
  seen(grid > 0 && D > 0 && (G == 1 || G == 2 || G == 4 || G == 8) && a.T > 0, "gated");
  return hipSuccess;
}
hipError_t launch_delta(int, int D, int G, int dk, const DeltaArgs& a, hipStream_t) {
  const int ns = a.nseg > 1 ? a.nseg : 1;
  seen(a.units > 0 && D > 0 && (G == 1 || G == 2 || G == 4 || G == 8) && dk >= 0 && dk <= 2 && a.T > 0 && a.seg_len > 0 &&
           (int64_t)(ns - 1) * a.seg_len < a.T && a.s_out && (a.out || a.s_out_all),
       "delta");
  return hipSuccess;
}
hipError_t launch_delta_compose(const float* M, const float* N, const float*, float* start, int units, int nseg, int D,
                                hipStream_t) {
  seen(M && N && start && units > 0 && nseg > 1 && (D == 32 || D == 64 || D == 128), "delta_compose");
  return hipSuccess;
}
hipError_t launch_eye(float* p, int D, hipStream_t) {
  seen(p && D > 0, "eye");
  return hipSuccess;
}
hipError_t launch_bwd_prep(int, const BwdArgs& a, hipStream_t) {
  seen(a.fq && a.fk && a.v32, "bwd_prep");
  return hipSuccess;
}
hipError_t launch_bwd_scan(const float* x, const float*, const float*, float* out, float*, int U, int T, int H, int D,
                           int, hipStream_t) {
  seen(x && out && U > 0 && T > 0 && H > 0 && D > 0, "bwd_scan");
  return hipSuccess;
}
hipError_t launch_bwd_dnum(int, const BwdArgs& a, hipStream_t) {
  seen(a.dnum != nullptr, "bwd_dnum");
  return hipSuccess;
}
hipError_t launch_bwd_dden(const BwdArgs& a, hipStream_t) {
  seen(a.dden != nullptr, "bwd_dden");
  return hipSuccess;
}
hipError_t launch_bwd_finish(int, const BwdArgs& a, hipStream_t) {
  seen(a.dq && a.dk && a.dv, "bwd_finish");
  return hipSuccess;
}
hipError_t launch_bwd_transpose(const float* in, float* out, int64_t U, int D, hipStream_t) {
  seen(in && out && U > 0 && D > 0, "bwd_transpose");
  return hipSuccess;
}
hipError_t launch_gated_step(int, int D, int G, const GatedStepArgs& a, hipStream_t) {
  seen(a.units > 0 && D > 0 && G > 0 && a.s_out, "gated_step");
  return hipSuccess;
}
hipError_t launch_delta_step(int, int D, int G, const GatedStepArgs& a, hipStream_t) {
  seen(a.units > 0 && D > 0 && G > 0 && a.s_out && a.beta, "delta_step");
  return hipSuccess;
}
hipError_t launch_gated_prefix(float* s, const float* av, const float*, int U, int nseg, int D, int, hipStream_t) {
  seen(s && av && U > 0 && nseg > 1 && D > 0, "gated_prefix");
  return hipSuccess;
}
hipError_t launch_gated_pd(int, int, int D, int G, const GatedArgs& a, int grid, hipStream_t) {
  seen(grid > 0 && D > 0 && G > 0 && a.T > 0, "gated_pd");
  return hipSuccess;
}
hipError_t launch_bwd_chunk(int pass, int io, int Dk, int Dv, int norm, const BwdChunkArgs& a, int grid,
                            hipStream_t) {
  seen(grid > 0 && pass >= 0 && pass <= 2 && (io == 1 || io == 2) && (Dk == 32 || Dk == 64) &&
           (Dv == 32 || Dv == 64) && a.nseg > 0 && a.seg_len % 32 == 0 && a.T > 0 && a.dy &&
           (!norm || (a.rden && a.dden)) && (pass == 2 || !a.fold || a.nseg <= kBwdFold),
       "bwd_chunk");
  return hipSuccess;
}
hipError_t launch_recur(int, int D, int G, int, int, const RecurArgs& a, hipStream_t) {
  seen(a.units > 0 && D == 128 && G > 0, "recur");
  return hipSuccess;
}
}  // namespace la

static int fails = 0;
static void expect(la_status got, la_status want, const char* what) {
  if (got != want) {
    printf("FAILED %s: got %s (%s), want %s\n", what, la_status_string(got), la_last_error_message(),
           la_status_string(want));
    ++fails;
  }
}
#define P(x) ((void*)(uintptr_t)(x))
#define F(x) ((float*)(uintptr_t)(x))

int main() {
  const uintptr_t G1 = (uintptr_t)1 << 36;  // fake buffers 64 GiB apart
  size_t n = 0;
  // forward: every path with valid arguments reaches its launches
  for (int causal = 0; causal < 2; ++causal)
    for (int dt = 0; dt < 3; ++dt)
      for (int64_t D : {32, 64, 128})
        for (int64_t Dv : {32, 64, 128})
          for (int64_t T : {0, 1, 63, 64, 200, 4096})
            for (int64_t BH : {1, 6, 512, 4096}) {
              expect(la_workspace_size(1, T, BH, D, Dv, dt, causal, &n), LA_OK, "workspace_size");
              const uintptr_t ws = n ? 9 * G1 : 0;
              expect(la_forward(P(G1), P(2 * G1), P(3 * G1), nullptr, causal ? F(4 * G1) : nullptr,
                                causal ? F(5 * G1) : nullptr, causal ? F(6 * G1) : nullptr,
                                causal ? F(7 * G1) : nullptr, causal, (int)(T % 2), 1, 1e-6f, P(8 * G1), 1, T, BH,
                                D, Dv, dt, P(ws), n, nullptr),
                     LA_OK, "forward");
            }
  // argument errors
  expect(la_forward(P(G1), P(2 * G1), P(3 * G1), nullptr, nullptr, nullptr, nullptr, nullptr, 1, 0, 1, 1e-6f,
                    P(G1 + 64), 2, 100, 4, 64, 64, 1, nullptr, 0, nullptr),
         LA_ERR_BAD_ARG, "out overlaps q");
  expect(la_forward(P(G1), P(2 * G1), P(3 * G1), nullptr, nullptr, nullptr, nullptr, nullptr, 1, 0, 1, -1.f, P(8 * G1),
                    2, 100, 4, 64, 64, 1, nullptr, 0, nullptr),
         LA_ERR_BAD_ARG, "negative eps");
  expect(la_forward(P(G1), P(2 * G1), P(3 * G1), nullptr, nullptr, nullptr, nullptr, nullptr, 1, 0, 1, 1e-6f,
                    P(8 * G1), (int64_t)1 << 40, 100, 4, 64, 64, 1, nullptr, 0, nullptr),
         LA_ERR_SHAPE, "sizes beyond the index range");
  expect(la_forward(P(G1), P(2 * G1), P(3 * G1), nullptr, nullptr, nullptr, nullptr, nullptr, 0, 1, 1, 1e-6f,
                    P(8 * G1), 8, 64, 128, 128, 128, 1, nullptr, 0, nullptr),
         LA_ERR_WORKSPACE, "non-causal without workspace");
  expect(la_forward_noalloc(P(G1), P(2 * G1), P(3 * G1), nullptr, nullptr, nullptr, nullptr, nullptr, 0, 1, 1, 1e-6f,
                            P(8 * G1), 8, 64, 128, 128, 128, 1, nullptr),
         LA_ERR_WORKSPACE, "noalloc beyond its scratch");
  // decode steps
  for (int dt = 0; dt < 3; ++dt)
    for (int64_t D : {32, 64, 128})
      for (int64_t Dv : {32, 64, 128})
        expect(la_step(P(G1), P(2 * G1), P(3 * G1), nullptr, F(4 * G1), F(5 * G1), F(4 * G1), F(5 * G1), 0, 1,
                       1e-6f, P(8 * G1), 256, 32, D, Dv, dt, nullptr),
               LA_OK, "step");
  // gated, per-dim, delta: any group size, every decay kind
  for (int dt = 0; dt < 3; ++dt)
    for (int64_t D : {32, 64, 128})
      for (int64_t Gq : {1, 3, 4, 8, 16, 32})
        for (int64_t T : {0, 1, 300, 32768})
          for (int pd = 0; pd < 2; ++pd) {
            const int64_t Hkv = 2, Hq = Hkv * Gq;
            expect(la_gated_workspace_size(1, T, Hq, Hkv, D, D, dt, pd, &n), LA_OK, "gated workspace");
            const uintptr_t ws = n ? 9 * G1 : 0;
            expect(la_gated_forward(P(G1), P(2 * G1), P(3 * G1), P(4 * G1), pd, nullptr, F(6 * G1), P(7 * G1), 1, T,
                                    Hq, Hkv, D, D, dt, 0.f, P(ws), n, nullptr),
                   LA_OK, "gated");
            expect(la_delta_workspace_size(1, T, Hq, Hkv, D, D, dt, pd, &n), LA_OK, "delta workspace");
            const uintptr_t dws = n ? 9 * G1 : 0;
            expect(la_delta_forward(P(G1), P(2 * G1), P(3 * G1), P(4 * G1), pd, P(5 * G1), 1, nullptr, F(6 * G1),
                                    P(7 * G1), 1, T, Hq, Hkv, D, D, dt, 0.f, P(dws), n, nullptr),
                   LA_OK, "delta");
            expect(la_gated_step(P(G1), P(2 * G1), P(3 * G1), P(4 * G1), pd, F(6 * G1), F(6 * G1), P(7 * G1), 3, Hq,
                                 Hkv, D, D, dt, 0.f, nullptr),
                   LA_OK, "gated step");
          }
  // backward: equal head sizes on every path; unequal ones (16-bit, 32 or 64)
  for (int dt = 0; dt < 3; ++dt)
    for (int64_t D : {32, 64, 128})
      for (int64_t Dv : {32, 64, 128})
        for (int64_t T : {0, 1, 150, 2048})
          for (int64_t BH : {3, 600})
            for (int norm = 0; norm < 2; ++norm) {
              const bool ok = D == Dv || (dt != 0 && D <= 64 && Dv <= 64);
              expect(la_backward_workspace_size(2, T, BH, D, Dv, dt, norm, &n), ok ? LA_OK : LA_ERR_UNSUPPORTED,
                     "backward workspace");
              expect(la_backward(P(G1), P(2 * G1), P(3 * G1), nullptr, nullptr, nullptr, P(4 * G1), nullptr, nullptr,
                                 0, norm, 1e-6f, P(5 * G1), P(6 * G1), P(7 * G1), F(8 * G1), norm ? F(9 * G1) : nullptr,
                                 2, T, BH, D, Dv, dt, P(10 * G1), ok ? n : 0, nullptr),
                     ok ? LA_OK : LA_ERR_UNSUPPORTED, "backward");
            }
  printf("%s: %d failures, %d launches (%d with bad arguments)\n", fails || bad ? "FAIL" : "OK", fails, launches,
         bad);
  return (fails || bad) ? 1 : 0;
}
