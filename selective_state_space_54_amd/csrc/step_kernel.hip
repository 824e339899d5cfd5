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
// are split over LPD adjacent lane-slots, NPL = min(N, 4) values each, so a
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

// Grid: blockIdx.y is the batch row; along x, each thread takes kSlots
// lane-slots of that row kStepBlock apart (every load instruction stays
// contiguous across the wavefront) and issues all their loads before any
// arithmetic, so several state loads per lane are in flight at once.  Row
// addressing needs only shifts (LPD is a power of two), no division.
constexpr int kSlots = 4;

template <int N, typename T, bool kZoh, bool kVec>
__global__ __launch_bounds__(kStepBlock) void selective_step_kernel(StepParams p) {
  constexpr int NPL = N < 4 ? N : 4;   // state values per lane-slot
  constexpr int LPD = N / NPL;         // lane-slots per channel: 1, 2, 4 or 8
  const int64_t b = blockIdx.y;
  const int64_t D = p.D;
  const int64_t total = D * LPD;       // lane-slots in this row
  const int64_t base = (int64_t)blockIdx.x * (kStepBlock * kSlots) + threadIdx.x;
  const int part = static_cast<int>(threadIdx.x % LPD);   // same for all of this lane's slots
  const int n0 = part * NPL;
  const T* xs = static_cast<const T*>(p.x) + b * D;
  const T* ds = static_cast<const T*>(p.delta) + b * D;
  float* hrow = p.h + b * D * N;
  float Bv[NPL], Cv[NPL];
  {
    const T* Bs = static_cast<const T*>(p.B) + b * N + n0;
    const T* Cs = static_cast<const T*>(p.C) + b * N + n0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      Bv[j] = to_float(Bs[j]);
      Cv[j] = to_float(Cs[j]);
    }
  }
  float hv[kSlots][NPL], av[kSlots][NPL], xv[kSlots], dv[kSlots];
#pragma unroll
  for (int s = 0; s < kSlots; ++s) {
    // a slot past the row's end re-reads the row's last channel (not stored)
    const int64_t slot = min(base + (int64_t)s * kStepBlock, total - LPD + part);
    const int64_t d = slot / LPD;
    load_f32<NPL, kVec>(hrow + d * N + n0, hv[s]);
    load_f32<NPL, kVec>(p.A + d * N + n0, av[s]);
    xv[s] = to_float(xs[d]);
    dv[s] = to_float(ds[d]);
  }
#pragma unroll
  for (int s = 0; s < kSlots; ++s) {
    const int64_t slot = base + (int64_t)s * kStepBlock;
    const int64_t d = slot / LPD;
    const float dx = dv[s] * xv[s];
    float yp = 0.0f;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const float abar = fast_exp2(dv[s] * (av[s][j] * kLog2e));
      float bx;
      if constexpr (kZoh) {
        const float u = xv[s] * Bv[j] / av[s][j];
        bx = __builtin_fmaf(abar, u, -u);        // (Abar - 1) / A * B * x
      } else {
        bx = dx * Bv[j];                         // delta B x
      }
      hv[s][j] = __builtin_fmaf(abar, hv[s][j], bx);
      yp = __builtin_fmaf(Cv[j], hv[s][j], yp);
    }
    // the lane-slots of one channel are adjacent lanes (LPD divides 64 and the
    // block), and all of them are past the end or none is
#pragma unroll
    for (int o = 1; o < LPD; o <<= 1) yp += __shfl_xor(yp, o, LPD);
    if (slot < total) {
      float* hp = hrow + d * N + n0;
      if constexpr (kVec && NPL == 4) {
        f32x4 u;
        u.x = hv[s][0]; u.y = hv[s][1]; u.z = hv[s][2]; u.w = hv[s][3];
        *reinterpret_cast<f32x4*>(hp) = u;
      } else {
#pragma unroll
        for (int j = 0; j < NPL; ++j) hp[j] = hv[s][j];
      }
      if (part == 0) {
        if (p.Dskip != nullptr) yp = __builtin_fmaf(p.Dskip[d], xv[s], yp);
        if (p.z != nullptr) yp *= silu(to_float(static_cast<const T*>(p.z)[b * D + d]));
        p.y[b * D + d] = yp;
      }
    }
  }
}

template <int N, typename T, bool kZoh>
hipError_t launch_step_t(const StepArgs& a, const StepParams& p, hipStream_t stream) {
  constexpr int NPL = N < 4 ? N : 4;
  constexpr int LPD = N / NPL;
  const int64_t row_slots = a.D * LPD;
  const dim3 grid((unsigned)((row_slots + kStepBlock * kSlots - 1) / (kStepBlock * kSlots)),
                  (unsigned)a.batch);
  const bool vec = NPL == 4 && reinterpret_cast<uintptr_t>(a.h) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(a.A) % 16 == 0;
  if (vec)
    hipLaunchKernelGGL((selective_step_kernel<N, T, kZoh, true>), grid, dim3(kStepBlock), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((selective_step_kernel<N, T, kZoh, false>), grid, dim3(kStepBlock), 0,
                       stream, p);
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
  StepParams p{a.x, a.delta, a.A, a.B, a.C, a.Dskip, a.z, a.h, a.y, a.D};
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
