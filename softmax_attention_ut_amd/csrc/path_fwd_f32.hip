// path_fwd (fp32 mode): blockwise PaTH attention forward in fp32 on the
// vector ALUs.  Intended for small shapes and for checking the blockwise
// algorithm at several chunk sizes; the bf16 MFMA kernel is the fast path.
//
// One workgroup owns query chunk a (C queries) of one head and scans the key
// chunks b = a, a-1, ..., 0 right to left (Dutch summary section 3,
// FlashAttention-style algorithm with a right-to-left scan):
//   b = a (diagonal):  logit_ij = q_i . k~_j + sum_{m>i} (q_i . w_m) Y[m][j]
//                      for j <= i; then the query is carried to the chunk
//                      start: q_i <- q_i - sum_{m<=i} (q_i . w_m) u_m
//   b < a:             logit_ij = q_i . k~_j;  then (if b > 0)
//                      q_i <- q_i - sum_m (q_i . w_m) u_m
// with k~, U, Y from path_ut.  The diagonal form follows from the full-matrix
// form lower(QK^T) - lower(QW^T) T^{-1} strictLower(WK^T) (Chinese notes,
// training strategy) and K~ = K - Y^T W.  Softmax is accumulated online
// (running max, running sum) in log2 units; the forget-gate bias
// sum_{s=j+1}^{i} log2 f_s is assembled from chunk-local sums.
#include "path_internal.h"

namespace path {

template <bool GATE>
__global__ __launch_bounds__(256) void path_fwd_f32_kernel(const FwdArgs a) {
    extern __shared__ float smem[];
    const int C = a.C, D = a.D, L = a.L, N = a.N;
    const int Lp = N * C;
    const int head = blockIdx.x / N, qa = blockIdx.x % N;
    const int tid = threadIdx.x;
    const int DP = D + 1, CP = C + 1;
    float* sQ = smem;             // [C][DP] query carried so far
    float* sO = sQ + C * DP;      // [C][DP] unnormalised output
    float* sS = sO + C * DP;      // [C][CP] logits, then probabilities
    float* sX = sS + C * CP;      // [C][CP] q . w_m
    float* sM = sX + C * CP;      // [C] running max (log2 units)
    float* sL = sM + C;           // [C] running sum
    float* sA = sL + C;           // [C] rescale factor of this step

    const float* q = static_cast<const float*>(a.q) + (size_t)head * L * D;
    const float* w = static_cast<const float*>(a.w) + (size_t)head * L * D;
    const float* v = static_cast<const float*>(a.v) + (size_t)head * L * D;
    const float* kt = static_cast<const float*>(a.kt) + (size_t)head * Lp * D;
    const float* ut = static_cast<const float*>(a.ut) + (size_t)head * Lp * D;
    const float* yt = static_cast<const float*>(a.yt) + (size_t)head * N * C * C;
    const float* loc = GATE ? a.loc + (size_t)head * Lp : nullptr;
    const float* csum = GATE ? a.csum + (size_t)head * N : nullptr;

    for (int idx = tid; idx < C * D; idx += 256) {
        const int i = idx / D, e = idx % D;
        const int p = qa * C + i;
        sQ[i * DP + e] = p < L ? q[(size_t)p * D + e] : 0.f;
        sO[i * DP + e] = 0.f;
    }
    for (int i = tid; i < C; i += 256) { sM[i] = -INFINITY; sL[i] = 0.f; }
    double dab = 0.0;   // sum of chunk gate sums between the query chunk and b
    __syncthreads();

    for (int b = qa; b >= 0; --b) {
        const bool diag = (b == qa);
        const int k0 = b * C;
        // X[i][m] = q_i . w_m ; S[i][j] = q_i . k~_j
        for (int idx = tid; idx < C * C; idx += 256) {
            const int i = idx / C, j = idx % C;
            const bool ok = k0 + j < L;
            float x = 0.f, s = 0.f;
            for (int e = 0; e < D; ++e) {
                const float qe = sQ[i * DP + e];
                x += qe * (ok ? w[(size_t)(k0 + j) * D + e] : 0.f);
                s += qe * kt[(size_t)(k0 + j) * D + e];
            }
            sX[i * CP + j] = x;
            sS[i * CP + j] = s;
        }
        __syncthreads();
        if (diag) {
            // S[i][j] += sum_{m>i} X[i][m] Y[m][j]
            const float* y = yt + (size_t)b * C * C;
            for (int idx = tid; idx < C * C; idx += 256) {
                const int i = idx / C, j = idx % C;
                float acc = 0.f;
                for (int m = i + 1; m < C; ++m) acc += sX[i * CP + m] * y[m * C + j];
                sS[i * CP + j] += acc;
            }
            __syncthreads();
        }
        // online softmax, one thread per row
        for (int i = tid; i < C; i += 256) {
            const float ai = GATE ? loc[qa * C + i] + (float)dab : 0.f;
            float mx = -INFINITY;
            const int jmax = diag ? i : C - 1;
            for (int j = 0; j <= jmax; ++j) {
                float z = sS[i * CP + j] * a.scale2;
                if (GATE) z += ai - loc[k0 + j];
                sS[i * CP + j] = z;
                mx = fmaxf(mx, z);
            }
            const float mnew = fmaxf(sM[i], mx);
            const float alpha = exp2f(sM[i] - mnew);
            float sum = 0.f;
            for (int j = 0; j < C; ++j) {
                const float p = (j <= jmax) ? exp2f(sS[i * CP + j] - mnew) : 0.f;
                sS[i * CP + j] = p;
                sum += p;
            }
            sM[i] = mnew;
            sL[i] = sL[i] * alpha + sum;
            sA[i] = alpha;
        }
        __syncthreads();
        // O = alpha O + P V ;  Q <- Q - X' U   (X' = lower part on the diagonal)
        for (int idx = tid; idx < C * D; idx += 256) {
            const int i = idx / D, e = idx % D;
            float o = sO[i * DP + e] * sA[i];
            for (int j = 0; j < C; ++j) {
                const int p = k0 + j;
                o += sS[i * CP + j] * (p < L ? v[(size_t)p * D + e] : 0.f);
            }
            sO[i * DP + e] = o;
            if (b > 0) {
                float qn = sQ[i * DP + e];
                const int mmax = diag ? i : C - 1;
                for (int m = 0; m <= mmax; ++m) qn -= sX[i * CP + m] * ut[(size_t)(k0 + m) * D + e];
                sQ[i * DP + e] = qn;
            }
        }
        if (GATE && b > 0) dab += (double)csum[b];
        __syncthreads();
    }
    float* out = static_cast<float*>(a.out) + (size_t)head * L * D;
    for (int idx = tid; idx < C * D; idx += 256) {
        const int i = idx / D, e = idx % D;
        const int p = qa * C + i;
        if (p < L) out[(size_t)p * D + e] = sO[i * DP + e] / sL[i];
    }
    if (a.lse)
        for (int i = tid; i < C; i += 256) {
            const int p = qa * C + i;
            if (p < L) a.lse[(size_t)head * L + p] = (sM[i] + log2f(sL[i])) * kLn2;
        }
}

hipError_t launch_path_fwd_f32(const FwdArgs& a, bool gate, hipStream_t s) {
    const dim3 grid(a.BH * a.N), block(256);
    const size_t smem = sizeof(float) * (size_t)(2 * a.C * (a.D + 1) + 2 * a.C * (a.C + 1) + 3 * a.C);
    if (gate) {
        hipFuncSetAttribute((const void*)path_fwd_f32_kernel<true>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        hipLaunchKernelGGL(path_fwd_f32_kernel<true>, grid, block, smem, s, a);
    } else {
        hipFuncSetAttribute((const void*)path_fwd_f32_kernel<false>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        hipLaunchKernelGGL(path_fwd_f32_kernel<false>, grid, block, smem, s, a);
    }
    return hipGetLastError();
}

}  // namespace path
