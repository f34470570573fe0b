// Internal declarations of the calibration-statistic code that follows the per-token
// top-k (not part of the ABI): co-occurrence counting on the GPU and the host-side
// similarity, spectral embedding and K-Means.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qe {

// Adds into cooc[n_dep][n_dep] (uint32) the number of tokens whose top-k lists (topk,
// int32 [T][k]) hold both token-dependent channels of each pair; slot[d_in] gives each
// channel's position among the token-dependent ones (entries outside [0, n_dep) and
// channels outside [0, d_in) are skipped).  ws: cooccur_workspace_bytes(T, n_dep) bytes,
// 16-byte aligned (the token masks).  Arguments are validated by the caller.
size_t cooccur_workspace_bytes(int T, int n_dep);
hipError_t launch_cooccur(const int32_t* topk, int T, int k, const int32_t* slot, int d_in, int n_dep,
                          uint32_t* cooc, void* ws, hipStream_t st);

// Host: frequency order of the channels (count descending, index ascending).
void frequency_order(const uint32_t* hist, int d_in, int32_t* order);

// Host: NPMI similarity -> normalized-Laplacian spectral embedding -> K-Means.
// Returns 0, or -1 when the eigenvalue iteration fails to converge.
// similarity [n][n], eigvals [n_clusters], embedding [n][n_clusters]: optional outputs.
int spectral_cluster(const uint32_t* cooc, int n, int64_t T, int n_clusters, double threshold, int32_t* labels,
                     double* similarity, double* eigvals, double* embedding);

// Host: eigenvalues (ascending) and orthonormal eigenvectors (columns of V, row-major
// [n][n]) of the symmetric matrix A [n][n] (row-major; overwritten).  Returns 0, or -1
// when the QR iteration fails to converge.
int symmetric_eigen(double* A, int n, double* eigvals, double* V);

}  // namespace qe
