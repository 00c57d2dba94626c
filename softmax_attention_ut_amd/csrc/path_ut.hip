// path_ut (fp32 mode): per-chunk UT transform of PaTH attention (gfx950),
// in fp32 on the vector ALUs.  The bf16 MFMA version is path_ut_bf16.hip.
//
// For chunk c (rows m = 0..C-1 = tokens c*C + m) the product of its
// transitions is held in the UT-transform form
//     H_{C-1} ... H_0 = I - W^T T^{-1} W,
//     T^{-1} = (I + strictLower(D W W^T))^{-1} D,   D = diag(beta)
// (Chinese notes, training strategy; Dutch summary section 3, UT transform).
// From it the kernel forms the per-chunk quantities the forward pass needs
// (the "boundary-adjusted" keys of the Dutch summary section 3):
//     U  = T^{-1} W                       query carried through the chunk:
//                                         q^T <- q^T - (q . W^T) U
//     Y  = T^{-1} strictLower(W K^T)      Y[m][j] for m > j
//     K~ = K - Y^T W                      k~_j = H_{C-1} ... H_{j+1} k_j
//     Z  = T^{-T} W   (cache hand-off)    key carried through the chunk:
//                                         k^T <- k^T - (k . W^T) Z
// T^{-1} is built row by row by forward substitution:
//     T^{-1}[m][:] = beta_m (e_m - sum_{p<m} G[m][p] T^{-1}[p][:]),  G = W W^T.
// Tokens past the sequence end are padded with w = 0, beta = 0 (H = I),
// k = v = 0 and log f = 0.
#include "path_internal.h"

namespace path {

template <typename T>
__device__ __forceinline__ float to_f(T x) { return static_cast<float>(x); }

__global__ __launch_bounds__(256) void path_ut_f32_kernel(const UtArgs a) {
    using Tin = float;
    extern __shared__ float smem[];
    const int C = a.C, D = a.D, L = a.L, N = a.N;
    const int Lp = N * C;
    const int head = blockIdx.x / N, c = blockIdx.x % N;
    const int p0 = c * C;
    const int tid = threadIdx.x;
    const int DP = D + 1, CP = C + 1;
    float* sW = smem;            // [C][DP]
    float* sK = sW + C * DP;     // [C][DP]
    float* sG = sK + C * DP;     // [C][CP]  G = W W^T, later R = strictLower(W K^T)
    float* sT = sG + C * CP;     // [C][CP]  T^{-1}
    float* sY = sT + C * CP;     // [C][CP]  Y
    float* sB = sY + C * CP;     // [C]      beta

    const Tin* w = static_cast<const Tin*>(a.w) + (size_t)head * L * D;
    const Tin* k = static_cast<const Tin*>(a.k) + (size_t)head * L * D;

    for (int idx = tid; idx < C * D; idx += 256) {
        const int m = idx / D, e = idx % D;
        const bool ok = p0 + m < L;
        sW[m * DP + e] = ok ? to_f(w[(size_t)(p0 + m) * D + e]) : 0.f;
        sK[m * DP + e] = ok ? to_f(k[(size_t)(p0 + m) * D + e]) : 0.f;
    }
    for (int m = tid; m < C; m += 256)
        sB[m] = (p0 + m < L) ? a.beta[(size_t)head * L + p0 + m] : 0.f;
    for (int idx = tid; idx < C * CP; idx += 256) sT[idx] = 0.f;
    __syncthreads();

    // G (strictly lower part only)
    for (int idx = tid; idx < C * C; idx += 256) {
        const int m = idx / C, n = idx % C;
        float g = 0.f;
        if (n < m)
            for (int e = 0; e < D; ++e) g += sW[m * DP + e] * sW[n * DP + e];
        sG[m * CP + n] = g;
    }
    __syncthreads();

    // T^{-1} by forward substitution: S lanes share one column n.
    {
        const int S = 256 / C;
        const int n = tid / S, sp = tid % S;
        for (int m = 0; m < C; ++m) {
            float part = 0.f;
            if (n < m)
                for (int p = n + sp; p < m; p += S) part += sG[m * CP + p] * sT[p * CP + n];
            for (int off = S >> 1; off > 0; off >>= 1) part += __shfl_xor(part, off, S);
            if (sp == 0 && n <= m) sT[m * CP + n] = sB[m] * ((n == m ? 1.f : 0.f) - part);
            __syncthreads();
        }
    }

    // R = strictLower(W K^T) into sG
    for (int idx = tid; idx < C * C; idx += 256) {
        const int n = idx / C, j = idx % C;
        float r = 0.f;
        if (n > j)
            for (int e = 0; e < D; ++e) r += sW[n * DP + e] * sK[j * DP + e];
        sG[n * CP + j] = r;
    }
    __syncthreads();

    // Y = T^{-1} R  (Y[m][j] = sum_{j<n<=m} T^{-1}[m][n] R[n][j])
    for (int idx = tid; idx < C * C; idx += 256) {
        const int m = idx / C, j = idx % C;
        float y = 0.f;
        for (int n = j + 1; n <= m; ++n) y += sT[m * CP + n] * sG[n * CP + j];
        sY[m * CP + j] = y;
    }
    __syncthreads();

    const size_t rowbase = (size_t)head * Lp + p0;         // row index into [BH][Lp]
    const size_t chunkbase = (size_t)head * N + c;         // chunk index into [BH][N]

    // K~[j][e] = K[j][e] - sum_{m>j} Y[m][j] W[m][e]
    for (int idx = tid; idx < C * D; idx += 256) {
        const int j = idx / D, s = idx % D;
        const int e = s;
        float x = sK[j * DP + e];
        for (int m = j + 1; m < C; ++m) x -= sY[m * CP + j] * sW[m * DP + e];
        static_cast<float*>(a.kt)[(rowbase + j) * D + s] = x;
    }
    // U = T^{-1} W
    for (int idx = tid; idx < C * D; idx += 256) {
        const int m = idx / D, e = idx % D;
        float u = 0.f;
        for (int n = 0; n <= m; ++n) u += sT[m * CP + n] * sW[n * DP + e];
        static_cast<float*>(a.ut)[(rowbase + m) * D + e] = u;
    }
    // Y out
    for (int idx = tid; idx < C * C; idx += 256) {
        const int m = idx / C, j = idx % C;
        static_cast<float*>(a.yt)[(chunkbase * C + m) * C + j] = sY[m * CP + j];
    }
    // Z = T^{-T} W  (only for the key-cache hand-off)
    if (a.zt) {
        for (int idx = tid; idx < C * D; idx += 256) {
            const int n = idx / D, e = idx % D;
            float z = 0.f;
            for (int m = n; m < C; ++m) z += sT[m * CP + n] * sW[m * DP + e];
            static_cast<float*>(a.zt)[(rowbase + n) * D + e] = z;
        }
    }
    // forget gate: chunk-local suffix sums (fp64), in log2 units
    if (a.loc && tid == 0) {
        double acc = 0.0;
        for (int s = C - 1; s >= 0; --s) {
            a.loc[rowbase + s] = static_cast<float>(-acc);
            const double lf = (p0 + s < L) ? (double)a.log_f[(size_t)head * L + p0 + s] : 0.0;
            acc += lf * 1.4426950408889634;
        }
        a.csum[chunkbase] = static_cast<float>(acc);
    }
}

static size_t ut_smem_bytes(int C, int D) {
    return sizeof(float) * (size_t)(2 * C * (D + 1) + 3 * C * (C + 1) + C);
}

hipError_t launch_path_ut_f32(const UtArgs& a, hipStream_t s) {
    const dim3 grid(a.BH * a.N), block(256);
    const size_t smem = ut_smem_bytes(a.C, a.D);
    hipFuncSetAttribute((const void*)path_ut_f32_kernel,
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    hipLaunchKernelGGL(path_ut_f32_kernel, grid, block, smem, s, a);
    return hipGetLastError();
}

}  // namespace path
