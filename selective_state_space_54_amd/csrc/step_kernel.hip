// One recurrent step of the selective SSM for every (batch row, channel): the
// constant-cost-per-token inference form ("Understanding Mamba", section 3.2
// and section 9.1, where each new token updates the fixed-size state once).
//
//   Abar = exp(delta A),  Bbar = delta B  (or (Abar - 1) / A * B, exact ZOH)
//   h    = Abar h + Bbar x                       (state updated in place)
//   y    = (C . h + Dskip x) * SiLU(z)           (feedthrough and gate optional)
//
// The step reads and writes the whole [batch, D, N] float32 state once, so it
// is bound by HBM bandwidth.  Layout on the lanes: a channel's N state values
// are split over LPD adjacent lanes, NPL = min(N, 4) values each, so a
// wavefront reads and writes contiguous 16-byte pieces of the state; the
// read-out sum over n is finished with a butterfly over those LPD lanes.
#include "mssm_internal.h"
#include "scan_device.h"

namespace mssm {

namespace {

constexpr int kStepBlock = 256;
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct StepParams {
  const void* x;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* Dskip;
  const void* z;
  float* h;
  float* y;
  int64_t chains;   // batch * D
  int64_t D;
};

template <int NPL, bool kVec>
__device__ __forceinline__ void load_f32(const float* p, float (&v)[NPL]) {
  if constexpr (kVec && NPL == 4) {
    const f32x4 u = *reinterpret_cast<const f32x4*>(p);
    v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
  } else {
#pragma unroll
    for (int j = 0; j < NPL; ++j) v[j] = p[j];
  }
}

template <int N, typename T, bool kZoh, bool kVec>
__global__ __launch_bounds__(kStepBlock) void selective_step_kernel(StepParams p) {
  constexpr int NPL = N < 4 ? N : 4;   // state values per lane
  constexpr int LPD = N / NPL;         // lanes per channel: 1, 2, 4 or 8
  const int64_t tid = (int64_t)blockIdx.x * kStepBlock + threadIdx.x;
  const int64_t g = tid / LPD;         // chain (b, d), row-major over [batch, D]
  const int part = static_cast<int>(tid % LPD);
  // LPD divides the block, so a chain's lanes leave together and every lane
  // that takes part in the butterfly below is active
  if (g >= p.chains) return;
  const int64_t b = g / p.D;
  const int64_t d = g - b * p.D;
  const int n0 = part * NPL;
  const T* xs = static_cast<const T*>(p.x);
  const T* ds = static_cast<const T*>(p.delta);
  const T* Bs = static_cast<const T*>(p.B) + b * N + n0;
  const T* Cs = static_cast<const T*>(p.C) + b * N + n0;
  const float xv = to_float(xs[g]);
  const float dv = to_float(ds[g]);
  float* hp = p.h + g * N + n0;
  float hv[NPL], av[NPL];
  load_f32<NPL, kVec>(hp, hv);
  load_f32<NPL, kVec>(p.A + d * N + n0, av);
  const float dx = dv * xv;
  float yp = 0.0f;
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const float Bn = to_float(Bs[j]);
    const float abar = fast_exp2(dv * (av[j] * kLog2e));
    float bx;
    if constexpr (kZoh) {
      const float u = xv * Bn / av[j];
      bx = __builtin_fmaf(abar, u, -u);          // (Abar - 1) / A * B * x
    } else {
      bx = dx * Bn;                              // delta B x
    }
    hv[j] = __builtin_fmaf(abar, hv[j], bx);
    yp = __builtin_fmaf(to_float(Cs[j]), hv[j], yp);
  }
#pragma unroll
  for (int o = 1; o < LPD; o <<= 1) yp += __shfl_xor(yp, o, LPD);
  if constexpr (kVec && NPL == 4) {
    f32x4 u;
    u.x = hv[0]; u.y = hv[1]; u.z = hv[2]; u.w = hv[3];
    *reinterpret_cast<f32x4*>(hp) = u;
  } else {
#pragma unroll
    for (int j = 0; j < NPL; ++j) hp[j] = hv[j];
  }
  if (part == 0) {
    if (p.Dskip != nullptr) yp = __builtin_fmaf(p.Dskip[d], xv, yp);
    if (p.z != nullptr) yp *= silu(to_float(static_cast<const T*>(p.z)[g]));
    p.y[g] = yp;
  }
}

template <int N, typename T, bool kZoh>
hipError_t launch_step_t(const StepArgs& a, const StepParams& p, hipStream_t stream) {
  constexpr int NPL = N < 4 ? N : 4;
  constexpr int LPD = N / NPL;
  const int64_t threads = p.chains * LPD;
  const int64_t grid = (threads + kStepBlock - 1) / kStepBlock;
  const bool vec = NPL == 4 && reinterpret_cast<uintptr_t>(a.h) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(a.A) % 16 == 0;
  if (vec)
    hipLaunchKernelGGL((selective_step_kernel<N, T, kZoh, true>), dim3((unsigned)grid),
                       dim3(kStepBlock), 0, stream, p);
  else
    hipLaunchKernelGGL((selective_step_kernel<N, T, kZoh, false>), dim3((unsigned)grid),
                       dim3(kStepBlock), 0, stream, p);
  return hipGetLastError();
}

template <int N>
hipError_t launch_step_n(const StepArgs& a, const StepParams& p, hipStream_t stream) {
  const bool zoh = a.bbar == MSSM_BBAR_ZOH;
  if (a.dtype == MSSM_FLOAT32)
    return zoh ? launch_step_t<N, float, true>(a, p, stream)
               : launch_step_t<N, float, false>(a, p, stream);
  return zoh ? launch_step_t<N, uint16_t, true>(a, p, stream)
             : launch_step_t<N, uint16_t, false>(a, p, stream);
}

}  // namespace

hipError_t launch_step(const StepArgs& a, hipStream_t stream) {
  StepParams p{a.x, a.delta, a.A, a.B, a.C, a.Dskip, a.z, a.h, a.y, a.batch * a.D, a.D};
  switch (a.N) {
    case 1: return launch_step_n<1>(a, p, stream);
    case 2: return launch_step_n<2>(a, p, stream);
    case 4: return launch_step_n<4>(a, p, stream);
    case 8: return launch_step_n<8>(a, p, stream);
    case 16: return launch_step_n<16>(a, p, stream);
    case 32: return launch_step_n<32>(a, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mssm
