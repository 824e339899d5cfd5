// Issue-rate and bandwidth probes for gfx950 (measurement only, not part of
// libmssm): the rates the scan's vector-ALU roof rests on.
//
// Each ALU probe runs `iters` iterations of a fixed instruction sequence
// written in inline assembly (so the compiler neither removes nor reorders
// it) over 16 independent registers per lane; the host times the launch and
// divides the instructions issued by the time.  One launch has enough
// wavefronts to give every SIMD several.
//   0  v_exp_f32         16 per iteration, each from a fixed input
//   1  v_fma_f32         16 dependent-per-register chains
//   2  v_mul_f32         16 per iteration
//   3  v_mul_f32 with a DPP row_newbcast operand (the single pass's broadcast)
//   4  the scan's per-element sequence, 16 elements per iteration:
//        t = delta * A2[n]; t = exp2(t); w = u * B[n]; h[n] = t h[n] + w;
//        y = C[n] h[n] + y            (4 single-rate VALU + 1 v_exp_f32)
//   5  read bandwidth: each thread sums 16-byte loads over a buffer (grid-stride)
// `out` receives one float per thread so no result is dead.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(256) void probe_exp(float* out, int64_t iters, float seed) {
  float in[16], o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    in[i] = seed * (i + 1) * 1e-3f + threadIdx.x * 1e-6f;
    o[i] = 0.0f;
  }
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) asm volatile("v_exp_f32 %0, %1" : "=v"(o[i]) : "v"(in[i]));
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += o[i];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void probe_fma(float* out, int64_t iters, float seed) {
  float acc[16];
  const float a = 0.999f, b = seed * 1e-3f;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = seed + i;
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      asm volatile("v_fma_f32 %0, %1, %0, %2" : "+v"(acc[i]) : "v"(a), "v"(b));
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += acc[i];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void probe_mul(float* out, int64_t iters, float seed) {
  float in[16], o[16];
  const float a = 0.999f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    in[i] = seed + i;
    o[i] = 0.0f;
  }
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i) asm volatile("v_mul_f32 %0, %1, %2" : "=v"(o[i]) : "v"(in[i]), "v"(a));
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += o[i];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// 16 multiplies whose first operand is lane 3 of the row (row_newbcast:3);
// the broadcast source is written before the loop and never again, and the
// block starts with the two wait states a DPP read needs after a VALU write.
__global__ __launch_bounds__(256) void probe_mul_dpp(float* out, int64_t iters, float seed) {
  float src = seed + threadIdx.x * 1e-3f;
  const float a = 0.999f;
  float o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = 0.0f;
  for (int64_t it = 0; it < iters; ++it) {
    asm volatile(
        "s_nop 1\n\t"
        "v_mul_f32_dpp %0, %16, %17 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %1, %16, %17 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %2, %16, %17 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %3, %16, %17 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %4, %16, %17 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %5, %16, %17 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %6, %16, %17 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %7, %16, %17 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %8, %16, %17 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %9, %16, %17 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %10, %16, %17 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %11, %16, %17 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %12, %16, %17 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %13, %16, %17 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %14, %16, %17 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_mul_f32_dpp %15, %16, %17 row_newbcast:3 row_mask:0xf bank_mask:0xf"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]),
          "=&v"(o[6]), "=&v"(o[7]), "=&v"(o[8]), "=&v"(o[9]), "=&v"(o[10]), "=&v"(o[11]),
          "=&v"(o[12]), "=&v"(o[13]), "=&v"(o[14]), "=&v"(o[15])
        : "v"(src), "v"(a));
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += o[i];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// The per-element sequence of the scan, 16 state indices per iteration.  A2
// in VGPRs (per lane), B and C as scalar operands (wave-uniform, as in the
// chunked kernels); delta and u vary per iteration so nothing is invariant.
__global__ __launch_bounds__(256) void probe_element(float* out, int64_t iters, float seed,
                                                     const float* __restrict__ bc) {
  float h[16], a2[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    h[i] = 0.0f;
    a2[i] = -1.4426950f * (i + 1);
  }
  // B and C held in SGPRs for the whole loop (read once, made uniform)
  int bs[16], cs[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) {
    bs[n] = __builtin_amdgcn_readfirstlane(__float_as_int(bc[n]));
    cs[n] = __builtin_amdgcn_readfirstlane(__float_as_int(bc[16 + n]));
  }
  float y = 0.0f, d = 1e-3f * seed + threadIdx.x * 1e-7f, u = 0.5f;
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      float t, w;
      asm volatile(
          "v_mul_f32 %0, %4, %5\n\t"
          "v_exp_f32 %0, %0\n\t"
          "v_mul_f32 %1, %6, %7\n\t"
          "v_fma_f32 %2, %0, %2, %1\n\t"
          "v_fma_f32 %3, %8, %2, %3"
          : "=&v"(t), "=&v"(w), "+v"(h[n]), "+v"(y)
          : "v"(d), "v"(a2[n]), "v"(u), "s"(bs[n]), "s"(cs[n]));
    }
    d += 1e-9f;
  }
  float s = y;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += h[i];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void probe_read(float* out, const uint4* __restrict__ buf,
                                                  int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
    const uint4 v = buf[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[blockIdx.x * 256 + threadIdx.x] = __uint_as_float(acc);
}

}  // namespace

extern "C" {

// Launch probe `which` (0-4: ALU, 5: read) on `stream` with `blocks` blocks of
// 256 threads; `out` holds blocks * 256 floats; `arg` is the read buffer
// (which = 5, n16 16-byte elements) or 32 floats of B and C (which = 4).
// Returns 0 on success, else the HIP error code.
int mssm_probe_launch(int which, int64_t blocks, int64_t iters, float* out, const void* arg,
                      int64_t n16, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 g(static_cast<unsigned>(blocks)), b(256);
  switch (which) {
    case 0: hipLaunchKernelGGL(probe_exp, g, b, 0, st, out, iters, 1.0f); break;
    case 1: hipLaunchKernelGGL(probe_fma, g, b, 0, st, out, iters, 1.0f); break;
    case 2: hipLaunchKernelGGL(probe_mul, g, b, 0, st, out, iters, 1.0f); break;
    case 3: hipLaunchKernelGGL(probe_mul_dpp, g, b, 0, st, out, iters, 1.0f); break;
    case 4:
      hipLaunchKernelGGL(probe_element, g, b, 0, st, out, iters, 1.0f,
                         static_cast<const float*>(arg));
      break;
    case 5:
      hipLaunchKernelGGL(probe_read, g, b, 0, st, out, static_cast<const uint4*>(arg), n16);
      break;
    default: return -1;
  }
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"
