// path_kcache: transformed key cache after a prefill of L tokens (gfx950).
//
// The inference form keeps every cached key already carried to "now":
// after token L-1 the cache holds H_{L-1} ... H_{j+1} k_j (Dutch summary
// section 3, "Inferentie"; Chinese notes, inference paragraph).  Per chunk
// b, path_ut gives k~_j = H_{end(b)} ... H_{j+1} k_j; this kernel carries
// every key chunk through each later chunk c = b+1 .. N-1 with the chunk's
// UT form, in row-vector form
//     k^T <- k^T - (k^T W_c^T) Z_c,    Z_c = T_c^{-T} W_c,
// which is (H_{end(c)} ... H_{start(c)}) k.  Layout and MFMA orientation are
// those of the query transport in path_fwd (the key rides in fp32
// accumulators, K^T -= Z^T X^T with X^T = W K^T; -Z^T comes from path_ut with
// its token axis in k-slot order and its d rows permuted, so the key's
// registers hold d in natural order).
#include "path_internal.h"

namespace path {

namespace {

__device__ __forceinline__ f32x16 mfma32k(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 pack8k(const f32x16& acc, int half) {
    bf16x8 r;
#pragma unroll
    for (int t = 0; t < 8; ++t) r[t] = static_cast<bf16>(acc[8 * half + t]);
    return r;
}

template <int C, int D, int PITCH>
__device__ __forceinline__ void stage_rows_k(bf16* dst, const bf16* src, int nvalid, int tid) {
    constexpr int UPR = D / 8;
#pragma unroll
    for (int u = tid; u < C * UPR; u += 256) {
        const int r = u / UPR, d0 = (u % UPR) * 8;
        uint4 val = {0u, 0u, 0u, 0u};
        if (r < nvalid) val = *reinterpret_cast<const uint4*>(src + (size_t)r * D + d0);
        *reinterpret_cast<uint4*>(dst + r * PITCH + d0) = val;
    }
}

template <int ROWS, int COLS, int PITCH>
__device__ __forceinline__ void stage_tile_k(bf16* dst, const bf16* src, int tid) {
    constexpr int UPR = COLS / 8;
    constexpr int UNITS = ROWS * UPR;
#pragma unroll
    for (int u = tid; u < UNITS; u += 256) {
        const int r = u / UPR, c8 = u % UPR;
        *reinterpret_cast<uint4*>(dst + r * PITCH + c8 * 8) =
            *reinterpret_cast<const uint4*>(src + (size_t)u * 8);
    }
}

}  // namespace

template <int D>
__global__ __launch_bounds__(256) void path_kcache_kernel(const KcacheArgs a) {
    constexpr int C = 64, PK = D + 8, PC = C + 8;
    constexpr int DT = D / 32, KSD = D / 16, KSC = C / 16;
    __shared__ __attribute__((aligned(16))) bf16 sW[C * PK];
    __shared__ __attribute__((aligned(16))) bf16 sZ[D * PC];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int L = a.L, N = a.N, Lp = N * C;
    const int nkb = (N + 1) / 2;
    // lightest work last: key block 0 carries its keys through the most chunks
    int head, kb;
    {
        const int bid = blockIdx.x;
        if ((a.BH & 7) == 0) {
            const int xcd = bid & 7, j = bid >> 3;
            head = xcd + 8 * (j / nkb);
            kb = j % nkb;
        } else {
            head = bid / nkb;
            kb = bid % nkb;
        }
    }
    const int kc_own = 2 * kb + (wave >> 1);
    const bool active = kc_own < N;
    const int jloc = (wave & 1) * 32 + l32;
    const int j = kc_own * C + jloc;

    const bf16* kt = static_cast<const bf16*>(a.kt) + (size_t)head * Lp * D;
    const bf16* win = static_cast<const bf16*>(a.w) + (size_t)head * L * D;
    const bf16* zt = static_cast<const bf16*>(a.zt) + (size_t)head * N * D * C;

    f32x16 kacc[DT];
    bf16x8 kB[KSD];
    if (active) {
        const bf16* krow = kt + (size_t)j * D;
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
            kB[ks] = *reinterpret_cast<const bf16x8*>(krow + 16 * ks + 8 * hh);
#pragma unroll
            for (int t = 0; t < 8; ++t) kacc[ks >> 1][8 * (ks & 1) + t] = static_cast<float>(kB[ks][t]);
        }
    }
    for (int c = 2 * kb + 1; c < N; ++c) {
        __syncthreads();
        stage_rows_k<C, D, PK>(sW, win + (size_t)c * C * D, min(C, L - c * C), tid);
        stage_tile_k<D, C, PC>(sZ, zt + (size_t)c * D * C, tid);
        __syncthreads();
        if (!active || c <= kc_own) continue;
        f32x16 x[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
            for (int v = 0; v < 16; ++v) x[k2][v] = 0.f;
            const bf16* aw = sW + (32 * k2 + l32) * PK + 8 * hh;
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks)
                x[k2] = mfma32k(*reinterpret_cast<const bf16x8*>(aw + 16 * ks), kB[ks], x[k2]);
        }
        bf16x8 xB[KSC];
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) xB[ks] = pack8k(x[ks >> 1], ks & 1);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const bf16* az = sZ + (32 * dt + l32) * PC + 8 * hh;
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks)
                kacc[dt] = mfma32k(*reinterpret_cast<const bf16x8*>(az + 16 * ks), xB[ks], kacc[dt]);
        }
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) kB[ks] = pack8k(kacc[ks >> 1], ks & 1);
    }
    if (!active || j >= L) return;
    // register 8s+t of kacc[dt] holds d = 32 dt + 16 s + 8 hh + t (the d rows
    // of -Z^T are stored permuted for this)
    const long long row = cache_row(a.map, head, j);
    if (row < 0) return;
    bf16* kout = static_cast<bf16*>(a.k_cache) + row * D;
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks)
        *reinterpret_cast<bf16x8*>(kout + 16 * ks + 8 * hh) = pack8k(kacc[ks >> 1], ks & 1);
    // values are copied unchanged, 4 bf16 per lane half
    const bf16* vin = static_cast<const bf16*>(a.v) + ((size_t)head * L + j) * D;
    bf16* vout = static_cast<bf16*>(a.v_cache) + row * D;
#pragma unroll
    for (int e = 4 * hh; e < D; e += 8)
        *reinterpret_cast<bf16x4*>(vout + e) = *reinterpret_cast<const bf16x4*>(vin + e);
}

hipError_t launch_path_kcache(const KcacheArgs& a, int D, hipStream_t s) {
    const dim3 grid(a.BH * ((a.N + 1) / 2)), block(256);
    if (D == 64) hipLaunchKernelGGL(path_kcache_kernel<64>, grid, block, 0, s, a);
    else if (D == 128) hipLaunchKernelGGL(path_kcache_kernel<128>, grid, block, 0, s, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace path
