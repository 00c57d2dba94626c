// path_ut (bf16 mode): per-chunk UT transform on gfx950 MFMA.
//
// Same quantities as the fp32 kernel in path_ut.hip (Chinese notes,
// training strategy: prod H = I - W^T T^{-1} W with
// T^{-1} = (I + strictLower(D W W^T))^{-1} D; Dutch summary section 3:
// boundary-adjusted keys computed per block beforehand), for chunks of
// C = 64 tokens and d in {64, 128}:
//     U  = T^{-1} W,   Y = T^{-1} strictLower(W K^T),   K~ = K - Y^T W,
//     Z  = T^{-T} W   (key-cache hand-off only)
// written in the operand layouts the scan kernel reads (see path_internal.h;
// permk = the k-slot permutation, applied to token axes and to the d rows of
// the transposed tiles):
//     kt [Lp][D]   K~ rows, natural
//     ut [N][D][C] -U^T:  ut[rho][sigma] = -U[permk(sigma)][permk(rho)]
//     vt [N][D][C]  V^T:  vt[rho][sigma] =  V[permk(sigma)][permk(rho)]
//     yt [N][C][C]  Y^T:  yt[j][sigma]   =  Y[permk(sigma)][j]
//     zt [N][D][C] -Z^T, laid out like ut (key-cache hand-off only)
//     mt [N][D][D] -M^T with M = W^T U (the chunk's product is I - M in
//                  row-vector form): mt[rho][d'] = -M[d'][permk(rho)]
//                  (optional; the d = 64 scan carries queries with it)
// plus the chunk-local forget-gate sums.
//
// Arithmetic.  G = W W^T and R = W K^T are bf16 MFMAs with fp32
// accumulation (exact products of the bf16 inputs).  T^{-1} is formed in
// fp32 by forward substitution, one lane per column,
//     T^{-1}[m][n] = beta_m (delta_mn - sum_{p<m} G[m][p] T^{-1}[p][n]),
// the column held in registers.  Products with the fp32 factors T^{-1}, R
// and Y use a two-term bf16 split x = hi + lo (hi = bf16(x),
// lo = bf16(x - hi)), so they carry ~16 significant bits before the final
// bf16 rounding of the stored result.
#include "path_internal.h"

namespace path {

namespace {

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void split8(const f32x16& acc, int half, float sign, bf16x8& hi,
                                       bf16x8& lo) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const float x = sign * acc[8 * half + t];
        const bf16 h = static_cast<bf16>(x);
        hi[t] = h;
        lo[t] = static_cast<bf16>(x - static_cast<float>(h));
    }
}

__device__ __forceinline__ bf16x8 ld8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ void zero(f32x16& a) {
#pragma unroll
    for (int v = 0; v < 16; ++v) a[v] = 0.f;
}

// bf16x8 from 8 consecutive accumulator registers, scaled
__device__ __forceinline__ bf16x8 cvt8(const f32x16& acc, int half, float sign) {
    bf16x8 r;
#pragma unroll
    for (int t = 0; t < 8; ++t) r[t] = static_cast<bf16>(sign * acc[8 * half + t]);
    return r;
}

}  // namespace

template <int D, bool WITH_Z>
__global__ __launch_bounds__(256) void path_ut_bf16_kernel(const UtArgs a) {
    constexpr int C = 64;
    constexpr int PW = D + 8;     // pitch of [token][d] tiles
    constexpr int PT = C + 8;     // pitch of [x][token-slot] bf16 tiles
    constexpr int GP = C + 4;     // pitch of the fp32 G rows
    constexpr int ET = D / 32;
    constexpr int KSD = D / 16;

    __shared__ __attribute__((aligned(16))) bf16 sW[C * PW];     // W rows, d natural
    __shared__ __attribute__((aligned(16))) bf16 sK[C * PW];     // K rows
    __shared__ __attribute__((aligned(16))) bf16 sWt[D * PT];    // W^T: [rho][sigma] = W[permk(sigma)][permk(rho)]
    __shared__ __attribute__((aligned(16))) bf16 sV[C * PW];     // V rows
    __shared__ __attribute__((aligned(16))) float sG[C * GP];    // G rows (p < m used)
    __shared__ __attribute__((aligned(16))) bf16 sTh[C * PT];    // T^{-1} rows, n in slots (hi)
    __shared__ __attribute__((aligned(16))) bf16 sTl[C * PT];    //                          (lo)
    __shared__ __attribute__((aligned(16))) bf16 sZh[WITH_Z ? C * PT : 8];  // T^{-T} rows, m slots
    __shared__ __attribute__((aligned(16))) bf16 sZl[WITH_Z ? C * PT : 8];
    __shared__ float sB[C];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int L = a.L, N = a.N, Lp = N * C;
    const int head = blockIdx.x / N, c = blockIdx.x % N;
    const int p0 = c * C;
    const int nvalid = min(C, L - p0);
    const size_t rowbase = (size_t)head * Lp + p0;
    const size_t chunkbase = (size_t)head * N + c;

    // ---- phase 0: stage W, K (rows), W^T (token slots), beta ----
    {
        const bf16* w = static_cast<const bf16*>(a.w) + ((size_t)head * L + p0) * D;
        const bf16* k = static_cast<const bf16*>(a.k) + ((size_t)head * L + p0) * D;
        const bf16* v = static_cast<const bf16*>(a.v) + ((size_t)head * L + p0) * D;
        constexpr int UPR = D / 8;
        for (int u = tid; u < C * UPR; u += 256) {
            const int r = u / UPR, d0 = (u % UPR) * 8;
            bf16x8 wv = {}, kv = {}, vv = {};
            if (r < nvalid) {
                wv = ld8(w + (size_t)r * D + d0);
                kv = ld8(k + (size_t)r * D + d0);
                vv = ld8(v + (size_t)r * D + d0);
            }
            *reinterpret_cast<bf16x8*>(sW + r * PW + d0) = wv;
            *reinterpret_cast<bf16x8*>(sK + r * PW + d0) = kv;
            *reinterpret_cast<bf16x8*>(sV + r * PW + d0) = vv;
            const int slot = permk(r);
#pragma unroll
            for (int e = 0; e < 8; ++e) sWt[permk(d0 + e) * PT + slot] = wv[e];
        }
        if (tid < C) sB[tid] = tid < nvalid ? a.beta[(size_t)head * L + p0 + tid] : 0.f;
    }
    __syncthreads();

    // ---- phase 1: G tiles (m-block >= p-block), accumulator rows p, cols m ----
    if (wave < 3) {
        const int mb = wave == 0 ? 0 : 1, pb = wave == 2 ? 1 : 0;
        f32x16 g;
        zero(g);
        const bf16* ap = sW + (32 * pb + l32) * PW + 8 * hh;
        const bf16* bp = sW + (32 * mb + l32) * PW + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) g = mfma(ld8(ap + 16 * ks), ld8(bp + 16 * ks), g);
        float* grow = sG + (32 * mb + l32) * GP + 32 * pb + 4 * hh;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            f32x4 v4 = {g[4 * r4], g[4 * r4 + 1], g[4 * r4 + 2], g[4 * r4 + 3]};
            *reinterpret_cast<f32x4*>(grow + 8 * r4) = v4;
        }
    }
    __syncthreads();

    // ---- phase 2: T^{-1} by forward substitution (wave 0, lane n = column n) ----
    if (wave == 0) {
        const int n = lane;
        const int sn = permk(n);
        float t[C];
#pragma unroll
        for (int m = 0; m < C; ++m) {
            float s = 0.f;
#pragma unroll
            for (int p = 0; p < (m & ~3); p += 4) {
                const f32x4 g4 = *reinterpret_cast<const f32x4*>(sG + m * GP + p);
                s = fmaf(g4[0], t[p], s);
                s = fmaf(g4[1], t[p + 1], s);
                s = fmaf(g4[2], t[p + 2], s);
                s = fmaf(g4[3], t[p + 3], s);
            }
#pragma unroll
            for (int p = (m & ~3); p < m; ++p) s = fmaf(sG[m * GP + p], t[p], s);
            const float tm = sB[m] * ((n == m ? 1.f : 0.f) - s);
            t[m] = tm;
            const bf16 h = static_cast<bf16>(tm);
            sTh[m * PT + sn] = h;
            sTl[m * PT + sn] = static_cast<bf16>(tm - static_cast<float>(h));
        }
        if (WITH_Z) {
            // row n of T^{-T} = column n of T^{-1}, token axis in slot order
#pragma unroll
            for (int s8 = 0; s8 < C; s8 += 8) {
                bf16x8 hi, lo;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = t[permk(s8 + e)];
                    hi[e] = static_cast<bf16>(x);
                    lo[e] = static_cast<bf16>(x - static_cast<float>(hi[e]));
                }
                *reinterpret_cast<bf16x8*>(sZh + n * PT + s8) = hi;
                *reinterpret_cast<bf16x8*>(sZl + n * PT + s8) = lo;
            }
        }
    } else {
        // waves 1-3: V^T tile, 8 token slots per 16-byte store
        bf16* vt = static_cast<bf16*>(a.vt) + chunkbase * D * C;
        for (int u = tid - 64; u < D * (C / 8); u += 192) {
            const int rho = u / (C / 8), s0 = (u % (C / 8)) * 8;
            const int e = permk(rho);
            bf16x8 col;
#pragma unroll
            for (int t = 0; t < 8; ++t) col[t] = sV[permk(s0 + t) * PW + e];
            *reinterpret_cast<bf16x8*>(vt + (size_t)rho * C + s0) = col;
        }
        if (tid == 64 && a.loc) {
            // forget gate: chunk-local suffix sums in log2 units (fp64)
            double acc = 0.0;
            for (int s = C - 1; s >= 0; --s) {
                a.loc[rowbase + s] = static_cast<float>(-acc);
                const double lf = s < nvalid ? (double)a.log_f[(size_t)head * L + p0 + s] : 0.0;
                acc += lf * 1.4426950408889634;
            }
            a.csum[chunkbase] = static_cast<float>(acc);
        }
    }
    __syncthreads();

    // ---- phase 3 ----
    if (wave < 2) {
        const int jt = wave;                 // key tile: columns j = 32 jt + l32
        const int j = 32 * jt + l32;
        // R[n][j] = w_n . k_j for n > j (accumulator rows n, cols j)
        f32x16 racc[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            zero(racc[nb]);
            const bf16* ap = sW + (32 * nb + l32) * PW + 8 * hh;
            const bf16* bp = sK + j * PW + 8 * hh;
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) racc[nb] = mfma(ld8(ap + 16 * ks), ld8(bp + 16 * ks), racc[nb]);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int nrow = 32 * nb + 8 * (v >> 2) + 4 * hh + (v & 3);
                if (nrow <= j) racc[nb][v] = 0.f;
            }
        }
        bf16x8 rh[4], rl[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) split8(racc[ks >> 1], ks & 1, 1.f, rh[ks], rl[ks]);
        // Y[m][j] = sum_n T^{-1}[m][n] R[n][j]
        f32x16 yacc[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            zero(yacc[mb]);
            const bf16* th = sTh + (32 * mb + l32) * PT + 8 * hh;
            const bf16* tl = sTl + (32 * mb + l32) * PT + 8 * hh;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 ah = ld8(th + 16 * ks), al = ld8(tl + 16 * ks);
                yacc[mb] = mfma(ah, rh[ks], yacc[mb]);
                yacc[mb] = mfma(ah, rl[ks], yacc[mb]);
                yacc[mb] = mfma(al, rh[ks], yacc[mb]);
            }
        }
        // store Y^T[j][m-slot]
        bf16* yrow = static_cast<bf16*>(a.yt) + (chunkbase * C + j) * C;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
                *reinterpret_cast<bf16x8*>(yrow + 32 * mb + 16 * s2 + 8 * hh) = cvt8(yacc[mb], s2, 1.f);
        // K~^T[d][j] = K^T[d][j] - sum_m W^T[d][m] Y[m][j]
        bf16x8 yh[4], yl[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) split8(yacc[ks >> 1], ks & 1, -1.f, yh[ks], yl[ks]);
        bf16* krow = static_cast<bf16*>(a.kt) + (rowbase + j) * D;
#pragma unroll
        for (int et = 0; et < ET; ++et) {
            // accumulator rows are sWt rows rho, i.e. d = permk(rho): register
            // 8s+t holds d = 32 et + 16 s + 8 hh + t
            f32x16 kacc;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const bf16x8 k8 = ld8(sK + j * PW + 32 * et + 16 * s2 + 8 * hh);
#pragma unroll
                for (int t = 0; t < 8; ++t) kacc[8 * s2 + t] = static_cast<float>(k8[t]);
            }
            const bf16* aw = sWt + (32 * et + l32) * PT + 8 * hh;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 w8 = ld8(aw + 16 * ks);
                kacc = mfma(w8, yh[ks], kacc);
                kacc = mfma(w8, yl[ks], kacc);
            }
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
                *reinterpret_cast<bf16x8*>(krow + 32 * et + 16 * s2 + 8 * hh) = cvt8(kacc, s2, 1.f);
        }
    } else {
        // waves 2, 3: U (and Z) for every token, a subset of the d columns
        for (int et = wave - 2; et < ET; et += 2) {
            const int e = 32 * et + l32;         // sWt row rho: d = permk(rho)
            const bf16* bw = sWt + e * PT + 8 * hh;
            // U[m][e] = sum_n T^{-1}[m][n] W[n][e]
            f32x16 uacc[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                zero(uacc[mt]);
                const bf16* th = sTh + (32 * mt + l32) * PT + 8 * hh;
                const bf16* tl = sTl + (32 * mt + l32) * PT + 8 * hh;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const bf16x8 w8 = ld8(bw + 16 * ks);
                    uacc[mt] = mfma(ld8(th + 16 * ks), w8, uacc[mt]);
                    uacc[mt] = mfma(ld8(tl + 16 * ks), w8, uacc[mt]);
                }
            }
            bf16* urow = static_cast<bf16*>(a.ut) + (chunkbase * D + e) * C;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
                    *reinterpret_cast<bf16x8*>(urow + 32 * mt + 16 * s2 + 8 * hh) = cvt8(uacc[mt], s2, -1.f);
            if (a.mt) {
                // M = W^T U (d x d): the whole chunk's transition product is
                // I - M in row-vector form.  The U accumulator's column is
                // d = permk(e), which is row e of -M^T in the stored layout
                // (row rho holds d = permk(rho)); columns d' come out natural.
                bf16x8 uh[4], ul[4];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) split8(uacc[ks >> 1], ks & 1, 1.f, uh[ks], ul[ks]);
                bf16* mrow = static_cast<bf16*>(a.mt) + (chunkbase * D + e) * D;
#pragma unroll
                for (int ot = 0; ot < ET; ++ot) {
                    f32x16 macc;
                    zero(macc);
                    const bf16* aw = sWt + (32 * ot + l32) * PT + 8 * hh;
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const bf16x8 w8 = ld8(aw + 16 * ks);
                        macc = mfma(w8, uh[ks], macc);
                        macc = mfma(w8, ul[ks], macc);
                    }
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2)
                        *reinterpret_cast<bf16x8*>(mrow + 32 * ot + 16 * s2 + 8 * hh) = cvt8(macc, s2, -1.f);
                }
            }
            if (WITH_Z) {
                // Z[n][e] = sum_m T^{-1}[m][n] W[m][e]
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    f32x16 zacc;
                    zero(zacc);
                    const bf16* zh = sZh + (32 * nt + l32) * PT + 8 * hh;
                    const bf16* zl = sZl + (32 * nt + l32) * PT + 8 * hh;
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const bf16x8 w8 = ld8(bw + 16 * ks);
                        zacc = mfma(ld8(zh + 16 * ks), w8, zacc);
                        zacc = mfma(ld8(zl + 16 * ks), w8, zacc);
                    }
                    bf16* zrow = static_cast<bf16*>(a.zt) + (chunkbase * D + e) * C;
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2)
                        *reinterpret_cast<bf16x8*>(zrow + 32 * nt + 16 * s2 + 8 * hh) = cvt8(zacc, s2, -1.f);
                }
            }
        }
    }
}

hipError_t launch_path_ut_bf16(const UtArgs& a, hipStream_t s) {
    const dim3 grid(a.BH * a.N), block(256);
    const bool z = a.zt != nullptr;
    if (a.D == 64) {
        if (z) hipLaunchKernelGGL((path_ut_bf16_kernel<64, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((path_ut_bf16_kernel<64, false>), grid, block, 0, s, a);
    } else if (a.D == 128) {
        if (z) hipLaunchKernelGGL((path_ut_bf16_kernel<128, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((path_ut_bf16_kernel<128, false>), grid, block, 0, s, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace path
