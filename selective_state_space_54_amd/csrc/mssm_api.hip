// C-ABI front end of the mssm library: argument checks, workspace, dispatch.
//
// Every check runs before the first HIP call, so argument errors come back on
// a machine without a GPU.  No static initialiser touches HIP.
#include <cstdio>
#include <cstring>
#include <limits>

#include "mssm_internal.h"

namespace {

thread_local char g_last_error[256] = "";

void set_hip_error(hipError_t e, const char* where) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d)", where, hipGetErrorString(e),
                static_cast<int>(e));
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a == 0 || b == 0) { *out = 0; return true; }
  if (a > std::numeric_limits<int64_t>::max() / b) return false;
  *out = a * b;
  return true;
}

// Shape checks shared by every scan entry point.
mssm_status check_shape(int64_t batch, int64_t L, int64_t D, int64_t N, mssm_dtype dtype) {
  if (batch < 0 || L < 0 || D < 0 || N < 0) return MSSM_ERROR_INVALID_VALUE;
  if (dtype != MSSM_FLOAT32 && dtype != MSSM_BFLOAT16) return MSSM_ERROR_INVALID_VALUE;
  if (!mssm::state_size_supported(N)) return MSSM_ERROR_NOT_SUPPORTED;
  int64_t bl, bld, bln, dn, bytes;
  if (!mul_ok(batch, L, &bl) || !mul_ok(bl, D, &bld) || !mul_ok(bl, N, &bln) ||
      !mul_ok(D, N, &dn) || !mul_ok(bld, 8, &bytes) || !mul_ok(bln, 8, &bytes) ||
      !mul_ok(dn, 8, &bytes))
    return MSSM_ERROR_SIZE_OVERFLOW;
  return MSSM_SUCCESS;
}

bool empty_problem(int64_t batch, int64_t L, int64_t D) { return batch == 0 || L == 0 || D == 0; }

mssm_status check_grid(const mssm::ScanPlan& p, int64_t batch, int64_t D, int64_t N) {
  if (p.chain) return MSSM_SUCCESS;   // sizes checked when the design was chosen
  // largest launch: chunk blocks (n_dtiles * K * batch) or carry blocks (n_dtiles * N * batch)
  const int64_t n_dtiles = (D + 255) / 256;
  int64_t blocks;
  const int64_t per_row = p.K > N ? static_cast<int64_t>(p.K) : N;
  if (!mul_ok(n_dtiles, per_row, &blocks) || !mul_ok(blocks, batch, &blocks))
    return MSSM_ERROR_SIZE_OVERFLOW;
  if (blocks * 256 > static_cast<int64_t>(std::numeric_limits<uint32_t>::max()))
    return MSSM_ERROR_NOT_SUPPORTED;
  return MSSM_SUCCESS;
}

}  // namespace

extern "C" {

int mssm_abi_version(void) { return MSSM_ABI_VERSION; }

const char* mssm_status_string(mssm_status s) {
  switch (s) {
    case MSSM_SUCCESS: return "success";
    case MSSM_ERROR_INVALID_VALUE: return "invalid value (null pointer, negative size or bad enum)";
    case MSSM_ERROR_NOT_SUPPORTED: return "not supported (state size, rank or grid outside the built kernels)";
    case MSSM_ERROR_SIZE_OVERFLOW: return "size overflow (an element count does not fit in int64)";
    case MSSM_ERROR_WORKSPACE: return "workspace missing or too small";
    case MSSM_ERROR_HIP: return "HIP error (see mssm_last_error_string)";
  }
  return "unknown status";
}

const char* mssm_last_error_string(void) { return g_last_error; }

int mssm_supports_state_size(int64_t N) { return mssm::state_size_supported(N) ? 1 : 0; }

mssm_status mssm_selective_scan_workspace_size(int64_t batch, int64_t L, int64_t D, int64_t N,
                                               mssm_dtype dtype, size_t* bytes) {
  if (!bytes) return MSSM_ERROR_INVALID_VALUE;
  const mssm_status s = check_shape(batch, L, D, N, dtype);
  if (s != MSSM_SUCCESS) return s;
  *bytes = empty_problem(batch, L, D) ? 0 : mssm::workspace_bound(batch, L, D, N);
  return MSSM_SUCCESS;
}

mssm_status mssm_selective_scan_fwd_ws(const void* x, const void* delta, const float* A,
                                       const void* B, const void* C, void* y, void* workspace,
                                       size_t workspace_bytes, int64_t batch, int64_t L,
                                       int64_t D, int64_t N, mssm_dtype dtype, void* stream) {
  mssm_status s = check_shape(batch, L, D, N, dtype);
  if (s != MSSM_SUCCESS) return s;
  if (empty_problem(batch, L, D)) return MSSM_SUCCESS;
  if (!x || !delta || !A || !B || !C || !y) return MSSM_ERROR_INVALID_VALUE;
  const mssm::ScanArgs a{x, delta, A, B, C, y, batch, L, D, N, dtype};
  const mssm::ScanPlan plan = mssm::plan_for(a);
  s = check_grid(plan, batch, D, N);
  if (s != MSSM_SUCCESS) return s;
  if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes))
    return MSSM_ERROR_WORKSPACE;
  const hipError_t e = mssm::launch_scan(a, plan, workspace, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    set_hip_error(e, "selective scan launch");
    return MSSM_ERROR_HIP;
  }
  return MSSM_SUCCESS;
}

mssm_status mssm_selective_scan_fwd(const void* x, const void* delta, const float* A,
                                    const void* B, const void* C, void* y, int64_t batch,
                                    int64_t L, int64_t D, int64_t N, mssm_dtype dtype,
                                    void* stream) {
  mssm_status s = check_shape(batch, L, D, N, dtype);
  if (s != MSSM_SUCCESS) return s;
  if (empty_problem(batch, L, D)) return MSSM_SUCCESS;
  if (!x || !delta || !A || !B || !C || !y) return MSSM_ERROR_INVALID_VALUE;
  const mssm::ScanArgs a{x, delta, A, B, C, y, batch, L, D, N, dtype};
  const mssm::ScanPlan plan = mssm::plan_for(a);
  s = check_grid(plan, batch, D, N);
  if (s != MSSM_SUCCESS) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (plan.workspace_bytes > 0) {
    const hipError_t e = hipMallocAsync(&ws, plan.workspace_bytes, st);
    if (e != hipSuccess) {
      set_hip_error(e, "workspace hipMallocAsync");
      return MSSM_ERROR_HIP;
    }
  }
  hipError_t e = mssm::launch_scan(a, plan, ws, st);
  if (ws) {
    const hipError_t f = hipFreeAsync(ws, st);
    if (e == hipSuccess) e = f;
  }
  if (e != hipSuccess) {
    set_hip_error(e, "selective scan launch");
    return MSSM_ERROR_HIP;
  }
  return MSSM_SUCCESS;
}

mssm_status mssm_selective_scan_fwd_noalloc(const void* x, const void* delta, const float* A,
                                            const void* B, const void* C, void* y,
                                            int64_t batch, int64_t L, int64_t D, int64_t N,
                                            mssm_dtype dtype, void* stream) {
  mssm_status s = check_shape(batch, L, D, N, dtype);
  if (s != MSSM_SUCCESS) return s;
  if (empty_problem(batch, L, D)) return MSSM_SUCCESS;
  if (!x || !delta || !A || !B || !C || !y) return MSSM_ERROR_INVALID_VALUE;
  const mssm::ScanArgs a{x, delta, A, B, C, y, batch, L, D, N, dtype};
  const mssm::ScanPlan plan = mssm::plan_for(a);
  s = check_grid(plan, batch, D, N);
  if (s != MSSM_SUCCESS) return s;
  if (plan.workspace_bytes > mssm::noalloc_scratch_bytes()) {
    std::snprintf(g_last_error, sizeof(g_last_error),
                  "chunk summaries need %zu bytes; the fixed scratch holds %zu",
                  plan.workspace_bytes, mssm::noalloc_scratch_bytes());
    return MSSM_ERROR_WORKSPACE;
  }
  // this device's copy of the fixed scratch array (its address is looked up
  // on the first call on each device)
  void* ws = nullptr;
  hipError_t e = mssm::scratch_pointer(&ws);
  if (e != hipSuccess) {
    set_hip_error(e, "scratch address");
    return MSSM_ERROR_HIP;
  }
  e = mssm::launch_scan(a, plan, plan.workspace_bytes > 0 ? ws : nullptr,
                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    set_hip_error(e, "selective scan launch");
    return MSSM_ERROR_HIP;
  }
  return MSSM_SUCCESS;
}

mssm_status mssm_selective_scan_fwd_ex(const void* x, const void* delta, const float* A,
                                       const void* B, const void* C, const float* Dskip,
                                       const void* z, const float* h0, float* y, float* h_last,
                                       mssm_bbar bbar, void* workspace, size_t workspace_bytes,
                                       int64_t batch, int64_t L, int64_t D, int64_t N,
                                       mssm_dtype dtype, void* stream) {
  mssm_status s = check_shape(batch, L, D, N, dtype);
  if (s != MSSM_SUCCESS) return s;
  if (bbar != MSSM_BBAR_EULER && bbar != MSSM_BBAR_ZOH) return MSSM_ERROR_INVALID_VALUE;
  if (batch == 0 || D == 0) return MSSM_SUCCESS;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (L == 0) {
    if (!h_last) return MSSM_SUCCESS;
    const hipError_t e = mssm::launch_state_init(h_last, h0, batch * D * N, st);
    if (e != hipSuccess) {
      set_hip_error(e, "state copy launch");
      return MSSM_ERROR_HIP;
    }
    return MSSM_SUCCESS;
  }
  if (!x || !delta || !A || !B || !C || !y) return MSSM_ERROR_INVALID_VALUE;
  mssm::ScanArgs a{x, delta, A, B, C, y, batch, L, D, N, dtype};
  a.Dskip = Dskip;
  a.z = z;
  a.h0 = h0;
  a.h_last = h_last;
  a.bbar = bbar;
  const mssm::ScanPlan plan = mssm::plan_for(a);
  s = check_grid(plan, batch, D, N);
  if (s != MSSM_SUCCESS) return s;
  if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes))
    return MSSM_ERROR_WORKSPACE;
  const hipError_t e = mssm::launch_scan(a, plan, workspace, st);
  if (e != hipSuccess) {
    set_hip_error(e, "selective scan launch");
    return MSSM_ERROR_HIP;
  }
  return MSSM_SUCCESS;
}

mssm_status mssm_selective_scan_step(const void* x, const void* delta, const float* A,
                                     const void* B, const void* C, const float* Dskip,
                                     const void* z, float* h, float* y, mssm_bbar bbar,
                                     int64_t batch, int64_t D, int64_t N, mssm_dtype dtype,
                                     void* stream) {
  mssm_status s = check_shape(batch, 1, D, N, dtype);
  if (s != MSSM_SUCCESS) return s;
  if (bbar != MSSM_BBAR_EULER && bbar != MSSM_BBAR_ZOH) return MSSM_ERROR_INVALID_VALUE;
  if (batch == 0 || D == 0) return MSSM_SUCCESS;
  if (!x || !delta || !A || !B || !C || !h || !y) return MSSM_ERROR_INVALID_VALUE;
  // grid: one row of blocks per batch row (at most 65535 rows), each row
  // covering D * (N / min(N, 4)) lane-slots
  if (batch > 65535) return MSSM_ERROR_NOT_SUPPORTED;
  const int64_t slots_per_chain = N < 4 ? 1 : N / 4;
  int64_t row_slots;
  if (!mul_ok(D, slots_per_chain, &row_slots)) return MSSM_ERROR_SIZE_OVERFLOW;
  if (row_slots > static_cast<int64_t>(std::numeric_limits<int32_t>::max()))
    return MSSM_ERROR_NOT_SUPPORTED;
  const mssm::StepArgs a{x, delta, A, B, C, Dskip, z, h, y, batch, D, N, dtype, bbar};
  const hipError_t e = mssm::launch_step(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    set_hip_error(e, "selective scan step launch");
    return MSSM_ERROR_HIP;
  }
  return MSSM_SUCCESS;
}

int mssm_fused_supports(int64_t N, int64_t R) {
  return (mssm::state_size_supported(N) && R >= 16 && R <= 1024 && R % 16 == 0) ? 1 : 0;
}

}  // extern "C"

namespace {

mssm_status check_fused(int64_t batch, int64_t L, int64_t D, int64_t N, int64_t R,
                        mssm_dtype dtype) {
  if (batch < 0 || L < 0 || D < 0 || N < 0 || R < 0) return MSSM_ERROR_INVALID_VALUE;
  if (dtype != MSSM_FLOAT32 && dtype != MSSM_BFLOAT16) return MSSM_ERROR_INVALID_VALUE;
  if (dtype != MSSM_BFLOAT16) return MSSM_ERROR_NOT_SUPPORTED;    // matrix cores take bf16
  if (!mssm_fused_supports(N, R)) return MSSM_ERROR_NOT_SUPPORTED;
  const mssm_status s = check_shape(batch, L, D, N, dtype);
  if (s != MSSM_SUCCESS) return s;
  int64_t m, t;
  if (!mul_ok(batch, L, &m) || !mul_ok(m, R + 2 * N, &t) || !mul_ok(t, 8, &t))
    return MSSM_ERROR_SIZE_OVERFLOW;
  if (m > std::numeric_limits<int32_t>::max() || D > std::numeric_limits<int32_t>::max())
    return MSSM_ERROR_NOT_SUPPORTED;                               // 32-bit GEMM sizes
  return MSSM_SUCCESS;
}

}  // namespace

extern "C" {

mssm_status mssm_selective_ssm_fused_workspace_size(int64_t batch, int64_t L, int64_t D,
                                                    int64_t N, int64_t R, mssm_dtype dtype,
                                                    size_t* bytes) {
  if (!bytes) return MSSM_ERROR_INVALID_VALUE;
  const mssm_status s = check_fused(batch, L, D, N, R, dtype);
  if (s != MSSM_SUCCESS) return s;
  *bytes = empty_problem(batch, L, D) ? 0 : mssm::fused_workspace_bound(batch, L, D, N, R);
  return MSSM_SUCCESS;
}

mssm_status mssm_selective_ssm_fused_fwd(const void* x, const void* W_xproj, const void* W_dtproj,
                                         const float* dt_bias, const float* A, float* y,
                                         void* workspace, size_t workspace_bytes, int64_t batch,
                                         int64_t L, int64_t D, int64_t N, int64_t R,
                                         mssm_dtype dtype, void* stream) {
  mssm_status s = check_fused(batch, L, D, N, R, dtype);
  if (s != MSSM_SUCCESS) return s;
  if (empty_problem(batch, L, D)) return MSSM_SUCCESS;
  if (!x || !W_xproj || !W_dtproj || !dt_bias || !A || !y) return MSSM_ERROR_INVALID_VALUE;
  const mssm::FusedPlan plan = mssm::plan_fused(batch, L, D, N, R, mssm::choose_fused_cpl(D),
                                                mssm::chain_fused_applies(batch, D, N, R, x, y));
  s = check_grid(plan.scan, batch, D, N);
  if (s != MSSM_SUCCESS) return s;
  if (!workspace || workspace_bytes < plan.workspace_bytes) return MSSM_ERROR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return MSSM_ERROR_WORKSPACE;
  const mssm::FusedArgs a{x, W_xproj, W_dtproj, dt_bias, A, y, batch, L, D, N, R};
  const mssm::FusedStatus st = mssm::launch_fused(a, plan, workspace,
                                                  static_cast<hipStream_t>(stream));
  if (st.blas_failed) {
    std::snprintf(g_last_error, sizeof(g_last_error), "rocBLAS x_proj GEMM failed");
    return MSSM_ERROR_HIP;
  }
  if (st.hip != hipSuccess) {
    set_hip_error(st.hip, "fused selective SSM launch");
    return MSSM_ERROR_HIP;
  }
  return MSSM_SUCCESS;
}

}  // extern "C"

namespace {

bool fits_grid(int64_t blocks) {
  return blocks <= static_cast<int64_t>(std::numeric_limits<uint32_t>::max());
}

mssm_status check_conv(int64_t batch, int64_t L, int64_t D, int64_t k, mssm_dtype dtype) {
  if (batch < 0 || L < 0 || D < 0 || k < 1) return MSSM_ERROR_INVALID_VALUE;
  if (dtype != MSSM_FLOAT32 && dtype != MSSM_BFLOAT16) return MSSM_ERROR_INVALID_VALUE;
  if (k > 8) return MSSM_ERROR_NOT_SUPPORTED;
  int64_t bl, bld, bytes;
  if (!mul_ok(batch, L, &bl) || !mul_ok(bl, D, &bld) || !mul_ok(bld, 8, &bytes))
    return MSSM_ERROR_SIZE_OVERFLOW;
  int64_t blocks;
  if (!mul_ok((D + 255) / 256, (L + 63) / 64, &blocks) || !mul_ok(blocks, batch, &blocks))
    return MSSM_ERROR_SIZE_OVERFLOW;
  if (!fits_grid(blocks)) return MSSM_ERROR_NOT_SUPPORTED;
  return MSSM_SUCCESS;
}

}  // namespace

extern "C" {

mssm_status mssm_causal_conv1d_silu(const void* u, const float* conv_w, const float* conv_b,
                                    float* out, int64_t batch, int64_t L, int64_t D, int64_t k,
                                    mssm_dtype dtype, void* stream) {
  const mssm_status s = check_conv(batch, L, D, k, dtype);
  if (s != MSSM_SUCCESS) return s;
  if (batch == 0 || L == 0 || D == 0) return MSSM_SUCCESS;
  if (!u || !conv_w || !out) return MSSM_ERROR_INVALID_VALUE;
  const hipError_t e = mssm::launch_conv1d_silu(u, dtype == MSSM_FLOAT32, conv_w, conv_b, out,
                                                nullptr, nullptr, batch, L, D,
                                                static_cast<int>(k),
                                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    set_hip_error(e, "causal conv1d launch");
    return MSSM_ERROR_HIP;
  }
  return MSSM_SUCCESS;
}

int mssm_mamba_block_supports(int64_t N, int64_t R, int64_t k) {
  return (mssm_fused_supports(N, R) && k >= 1 && k <= 8) ? 1 : 0;
}

}  // extern "C"

namespace {

mssm_status check_block(int64_t batch, int64_t L, int64_t Dm, int64_t Di, int64_t N, int64_t R,
                        int64_t k, mssm_dtype dtype) {
  if (Dm < 0 || k < 1) return MSSM_ERROR_INVALID_VALUE;
  mssm_status s = check_fused(batch, L, Di, N, R, dtype);
  if (s != MSSM_SUCCESS) return s;
  s = check_conv(batch, L, Di, k, dtype);
  if (s != MSSM_SUCCESS) return s;
  int64_t m, t;
  if (!mul_ok(batch, L, &m) || !mul_ok(m, Dm, &t) || !mul_ok(t, 8, &t) ||
      !mul_ok(m, Di, &t) || !mul_ok(t, 24, &t))
    return MSSM_ERROR_SIZE_OVERFLOW;
  if (Dm > std::numeric_limits<int32_t>::max() || 2 * Di > std::numeric_limits<int32_t>::max())
    return MSSM_ERROR_NOT_SUPPORTED;                               // 32-bit GEMM sizes
  return MSSM_SUCCESS;
}

}  // namespace

extern "C" {

mssm_status mssm_mamba_block_workspace_size(int64_t batch, int64_t L, int64_t Dm, int64_t Di,
                                            int64_t N, int64_t R, int64_t k, mssm_dtype dtype,
                                            size_t* bytes) {
  if (!bytes) return MSSM_ERROR_INVALID_VALUE;
  const mssm_status s = check_block(batch, L, Dm, Di, N, R, k, dtype);
  if (s != MSSM_SUCCESS) return s;
  *bytes = (batch == 0 || L == 0 || Di == 0 || Dm == 0)
               ? 0
               : mssm::block_workspace_bound(batch, L, Dm, Di, N, R);
  return MSSM_SUCCESS;
}

mssm_status mssm_mamba_block_fwd(const void* u0, const void* W_in, const float* conv_w,
                                 const float* conv_b, const void* W_x, const void* W_dt,
                                 const float* dt_bias, const float* A, const float* Dskip,
                                 const void* W_out, float* out, void* workspace,
                                 size_t workspace_bytes, int64_t batch, int64_t L, int64_t Dm,
                                 int64_t Di, int64_t N, int64_t R, int64_t k, mssm_dtype dtype,
                                 void* stream) {
  mssm_status s = check_block(batch, L, Dm, Di, N, R, k, dtype);
  if (s != MSSM_SUCCESS) return s;
  if (batch == 0 || L == 0 || Dm == 0) return MSSM_SUCCESS;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!out) return MSSM_ERROR_INVALID_VALUE;
  if (Di == 0) {   // an empty inner dimension: the output projection sums nothing
    const hipError_t e = mssm::launch_state_init(out, nullptr, batch * L * Dm, st);
    if (e != hipSuccess) {
      set_hip_error(e, "zero fill launch");
      return MSSM_ERROR_HIP;
    }
    return MSSM_SUCCESS;
  }
  if (!u0 || !W_in || !conv_w || !W_x || !W_dt || !dt_bias || !A || !W_out)
    return MSSM_ERROR_INVALID_VALUE;
  // the block's scan reads and writes its own workspace buffers (256-byte aligned)
  const mssm::BlockPlan plan =
      mssm::plan_block(batch, L, Dm, Di, N, R, mssm::choose_fused_cpl(Di),
                       mssm::chain_fused_applies(batch, Di, N, R, workspace, workspace));
  s = check_grid(plan.scan, batch, Di, N);
  if (s != MSSM_SUCCESS) return s;
  if (!workspace || workspace_bytes < plan.workspace_bytes) return MSSM_ERROR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return MSSM_ERROR_WORKSPACE;
  const mssm::BlockArgs a{u0, W_in, conv_w, conv_b, W_x, W_dt, dt_bias, A, Dskip, W_out, out,
                          batch, L, Dm, Di, N, R, static_cast<int>(k)};
  const mssm::FusedStatus r = mssm::launch_block(a, plan, workspace, st);
  if (r.blas_failed) {
    std::snprintf(g_last_error, sizeof(g_last_error), "rocBLAS projection GEMM failed");
    return MSSM_ERROR_HIP;
  }
  if (r.hip != hipSuccess) {
    set_hip_error(r.hip, "Mamba block launch");
    return MSSM_ERROR_HIP;
  }
  return MSSM_SUCCESS;
}

}  // extern "C"

namespace {

// The backward call; with_saved: the checkpoints (and y_pre with the gate)
// come from `saved`, written by mssm_selective_scan_fwd_save.
mssm_status bwd_impl(const void* x, const void* delta, const float* A, const void* B,
                     const void* C, const float* Dskip, const void* z, const float* h0,
                     const float* dout, float* dx, float* ddelta, float* dA, float* dB,
                     float* dC, float* dDskip, float* dz, float* dh0, const float* saved,
                     size_t saved_bytes, bool with_saved, void* workspace,
                     size_t workspace_bytes, int64_t batch, int64_t L, int64_t D, int64_t N,
                     mssm_dtype dtype, void* stream) {
  mssm_status s = check_shape(batch, L, D, N, dtype);
  if (s != MSSM_SUCCESS) return s;
  if ((Dskip != nullptr) != (dDskip != nullptr) || (z != nullptr) != (dz != nullptr))
    return MSSM_ERROR_INVALID_VALUE;       // each optional input comes with its gradient
  if (dh0 != nullptr && h0 == nullptr) return MSSM_ERROR_INVALID_VALUE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (D > 0 && !dA) return MSSM_ERROR_INVALID_VALUE;
  if (batch == 0 || L == 0 || D == 0) {
    // nothing flows back: the gradients that still have elements are zero
    hipError_t e = hipSuccess;
    if (D > 0) e = mssm::launch_state_init(dA, nullptr, D * N, st);
    if (e == hipSuccess && dDskip && D > 0) e = mssm::launch_state_init(dDskip, nullptr, D, st);
    if (e == hipSuccess && dh0 && D > 0) e = mssm::launch_state_init(dh0, nullptr, batch * D * N, st);
    if (e == hipSuccess && D == 0 && batch * L > 0) {
      if (!dB || !dC) return MSSM_ERROR_INVALID_VALUE;
      e = mssm::launch_state_init(dB, nullptr, batch * L * N, st);
      if (e == hipSuccess) e = mssm::launch_state_init(dC, nullptr, batch * L * N, st);
    }
    if (e != hipSuccess) {
      set_hip_error(e, "zero fill launch");
      return MSSM_ERROR_HIP;
    }
    return MSSM_SUCCESS;
  }
  if (!x || !delta || !A || !B || !C || !dout || !dx || !ddelta || !dB || !dC)
    return MSSM_ERROR_INVALID_VALUE;
  mssm::BwdArgs a{x,  delta,  A,  B,  C,      Dskip, z,  h0,  dout,  dx,    ddelta, dA,
                  dB, dC,     dDskip, dz, dh0, batch, L, D, N, dtype};
  bool chain;
  if (with_saved) {
    if (N != 16 || D % 16 != 0) return MSSM_ERROR_NOT_SUPPORTED;
    if (!saved) return MSSM_ERROR_INVALID_VALUE;
    const mssm::SavedLayout lay = mssm::saved_layout(batch, L, D, N, z != nullptr);
    if (saved_bytes < lay.bytes || reinterpret_cast<uintptr_t>(saved) % 256 != 0)
      return MSSM_ERROR_WORKSPACE;
    const char* base = reinterpret_cast<const char*>(saved);
    a.saved_ck = reinterpret_cast<const float*>(base + lay.ck_offset);
    a.saved_y_pre = z ? reinterpret_cast<const float*>(base + lay.y_pre_offset) : nullptr;
    if (!mssm::chain_bwd_layout_ok(a)) return MSSM_ERROR_NOT_SUPPORTED;
    chain = true;
  } else {
    chain = mssm::chain_bwd_applies(a);
  }
  const mssm::BwdPlan plan = mssm::plan_bwd(batch, L, D, N, chain);
  if (!plan.chain) {
    const int64_t n_dtiles = (D + 255) / 256;
    int64_t blocks;
    if (!mul_ok(n_dtiles, plan.K, &blocks) || !mul_ok(blocks, batch, &blocks))
      return MSSM_ERROR_SIZE_OVERFLOW;
    if (blocks > static_cast<int64_t>(std::numeric_limits<uint32_t>::max()) / 256 ||
        plan.K > 65535)
      return MSSM_ERROR_NOT_SUPPORTED;
  }
  if (!workspace || workspace_bytes < plan.workspace_bytes) return MSSM_ERROR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return MSSM_ERROR_WORKSPACE;
  const hipError_t e = mssm::launch_bwd(a, plan, workspace, st);
  if (e != hipSuccess) {
    set_hip_error(e, "selective scan backward launch");
    return MSSM_ERROR_HIP;
  }
  return MSSM_SUCCESS;
}

}  // namespace

extern "C" {

mssm_status mssm_selective_scan_bwd_workspace_size(int64_t batch, int64_t L, int64_t D, int64_t N,
                                                   mssm_dtype dtype, size_t* bytes) {
  if (!bytes) return MSSM_ERROR_INVALID_VALUE;
  const mssm_status s = check_shape(batch, L, D, N, dtype);
  if (s != MSSM_SUCCESS) return s;
  *bytes = (batch == 0 || L == 0 || D == 0) ? 0 : mssm::bwd_workspace_bound(batch, L, D, N);
  return MSSM_SUCCESS;
}

mssm_status mssm_selective_scan_bwd(const void* x, const void* delta, const float* A,
                                    const void* B, const void* C, const float* Dskip,
                                    const void* z, const float* h0, const float* dout, float* dx,
                                    float* ddelta, float* dA, float* dB, float* dC, float* dDskip,
                                    float* dz, float* dh0, void* workspace, size_t workspace_bytes,
                                    int64_t batch, int64_t L, int64_t D, int64_t N,
                                    mssm_dtype dtype, void* stream) {
  return bwd_impl(x, delta, A, B, C, Dskip, z, h0, dout, dx, ddelta, dA, dB, dC, dDskip, dz, dh0,
                  nullptr, 0, false, workspace, workspace_bytes, batch, L, D, N, dtype, stream);
}

mssm_status mssm_selective_scan_saved_size(int64_t batch, int64_t L, int64_t D, int64_t N,
                                           int gate, size_t* bytes) {
  if (!bytes) return MSSM_ERROR_INVALID_VALUE;
  const mssm_status s = check_shape(batch, L, D, N, MSSM_FLOAT32);
  if (s != MSSM_SUCCESS) return s;
  *bytes = mssm::saved_layout(batch, L, D, N, gate != 0).bytes;
  return MSSM_SUCCESS;
}

mssm_status mssm_selective_scan_fwd_save(const void* x, const void* delta, const float* A,
                                         const void* B, const void* C, const float* Dskip,
                                         const void* z, const float* h0, float* y,
                                         float* h_last, float* saved, size_t saved_bytes,
                                         int64_t batch, int64_t L, int64_t D, int64_t N,
                                         mssm_dtype dtype, void* stream) {
  mssm_status s = check_shape(batch, L, D, N, dtype);
  if (s != MSSM_SUCCESS) return s;
  if (batch == 0 || D == 0) return MSSM_SUCCESS;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (L == 0) {   // nothing to save; the state passes through
    if (!h_last) return MSSM_SUCCESS;
    const hipError_t e = mssm::launch_state_init(h_last, h0, batch * D * N, st);
    if (e != hipSuccess) {
      set_hip_error(e, "state copy launch");
      return MSSM_ERROR_HIP;
    }
    return MSSM_SUCCESS;
  }
  if (N != 16 || D % 16 != 0) return MSSM_ERROR_NOT_SUPPORTED;
  if (!x || !delta || !A || !B || !C || !y || !saved) return MSSM_ERROR_INVALID_VALUE;
  const mssm::SavedLayout lay = mssm::saved_layout(batch, L, D, N, z != nullptr);
  if (saved_bytes < lay.bytes || reinterpret_cast<uintptr_t>(saved) % 256 != 0)
    return MSSM_ERROR_WORKSPACE;
  mssm::ScanArgs a{x, delta, A, B, C, y, batch, L, D, N, dtype};
  a.Dskip = Dskip;
  a.z = z;
  a.h0 = h0;
  a.h_last = h_last;
  if (!mssm::chain_layout_ok(a)) return MSSM_ERROR_NOT_SUPPORTED;
  char* base = reinterpret_cast<char*>(saved);
  float* ck = reinterpret_cast<float*>(base + lay.ck_offset);
  float* y_pre = z ? reinterpret_cast<float*>(base + lay.y_pre_offset) : nullptr;
  const hipError_t e = mssm::launch_chain_save(a, ck, y_pre, st);
  if (e != hipSuccess) {
    set_hip_error(e, "selective scan (saving) launch");
    return MSSM_ERROR_HIP;
  }
  return MSSM_SUCCESS;
}

mssm_status mssm_selective_scan_bwd_saved(const void* x, const void* delta, const float* A,
                                          const void* B, const void* C, const float* Dskip,
                                          const void* z, const float* h0, const float* saved,
                                          size_t saved_bytes, const float* dout, float* dx,
                                          float* ddelta, float* dA, float* dB, float* dC,
                                          float* dDskip, float* dz, float* dh0, void* workspace,
                                          size_t workspace_bytes, int64_t batch, int64_t L,
                                          int64_t D, int64_t N, mssm_dtype dtype, void* stream) {
  return bwd_impl(x, delta, A, B, C, Dskip, z, h0, dout, dx, ddelta, dA, dB, dC, dDskip, dz, dh0,
                  saved, saved_bytes, true, workspace, workspace_bytes, batch, L, D, N, dtype,
                  stream);
}

}  // extern "C"
