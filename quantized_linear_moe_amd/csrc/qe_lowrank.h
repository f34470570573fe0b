// Internal declarations of the expert construction (not part of the ABI): the weight
// quantization error, whitening weights from calibration activations, and the randomized
// truncated SVD that turns them into the low-rank factors of the shared and routed experts.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qe {

// E = W_f - diag(s_w) q diag(1/s) with the weight quantizer's codes (device, [d_out][d_in]).
hipError_t launch_quant_error(const float* W_f, const float* s, int d_out, int d_in, int w_bits, float* E,
                              hipStream_t st);

// c[j] = sqrt(mean_t x[t][j]^2) (double sums; ws: channel_rms_workspace_bytes(T, d_in) bytes).
size_t channel_rms_workspace_bytes(int T, int d_in);
hipError_t launch_channel_rms(const void* x, int x_dtype, int T, int d_in, float* c, void* ws, hipStream_t st);

// E[i][j] -= sum_l A[j][l] B[l][i]  (A [d_in][r], B [r][d_out], device float32, r <= 64).
hipError_t launch_sub_lowrank(float* E, int d_out, int d_in, const float* A, const float* B, int r, hipStream_t st);

// Randomized truncated SVD of M = diag(w) E^T (host-orchestrated, synchronizes `st`): see
// lowrank_fit in k_lowrank.hip.  A [d_in][rank], B [rank][d_out], sigma [rank]: host outputs.
// Returns hipSuccess, or the first HIP error.
size_t lowrank_workspace_bytes(int d_out, int d_in, int k);
hipError_t lowrank_fit(const float* E, int d_out, int d_in, const float* w, const float* omega, int k, int rank,
                       int power_iters, float* A, float* B, double* sigma, void* ws, hipStream_t st);

// SE and REs of one linear (see build_experts in k_lowrank.hip); arguments validated by the caller.
size_t build_experts_workspace_bytes(int d_out, int d_in, int k, int r_max);
hipError_t build_experts(const float* W_f, const float* s, int d_out, int d_in, int w_bits, const float* c,
                         const int32_t* dep, const int32_t* labels, int n_dep, int n_r, int r_s, int r_r,
                         const float* omegas, int k, int power_iters, float* A_s, float* B_s, float* A_r, float* B_r,
                         double* sigma_s, double* sigma_r, void* ws, hipStream_t st);

// Covariance-whitened fit of E diag(mask) on the calibration tokens X (device float32 [T][d_in];
// mask device float32 0/1 [d_in] or NULL; omega device [T][k]): A [d_in][rank], B [rank][d_out],
// sigma [rank] host outputs (see lowrank_fit_cov in k_lowrank.hip).  Synchronizes `st`.
size_t lowrank_cov_workspace_bytes(int d_out, int d_in, int T, int k);
hipError_t lowrank_fit_cov(const float* E, int d_out, int d_in, const float* X, int T, const float* mask,
                           const float* omega, int k, int rank, int power_iters, float* A, float* B, double* sigma,
                           void* ws, hipStream_t st);
size_t build_experts_cov_workspace_bytes(int d_out, int d_in, int T, int k, int r_max);
hipError_t build_experts_cov(const float* W_f, const float* s, int d_out, int d_in, int w_bits, const void* x,
                             int x_dtype, int T, const int32_t* dep, const int32_t* labels, int n_dep, int n_r,
                             int r_s, int r_r, const float* omegas, int k, int power_iters, float* A_s, float* B_s,
                             float* A_r, float* B_r, double* sigma_s, double* sigma_r, void* ws, hipStream_t st);

// Router: per-token targets mean_i |x_t (E_1^T - A_g B_g)|_i and the ridge least-squares fit of
// R to them (see router_targets / router_fit in k_lowrank.hip); arguments validated by the caller.
size_t router_targets_workspace_bytes(int d_out, int d_in, int n_r, int r_r);
hipError_t router_targets(const float* E1, int d_out, int d_in, const void* x, int x_dtype, int T, const float* A_r,
                          const float* B_r, int n_r, int r_r, float* target, void* ws, hipStream_t st);
size_t router_fit_workspace_bytes(int T, int d_in, int n_r);
hipError_t router_fit(const void* x, int x_dtype, int T, int d_in, const float* target, int n_r, double ridge,
                      int max_iters, double tol, float* R, int* iters_done, void* ws, hipStream_t st);

}  // namespace qe
