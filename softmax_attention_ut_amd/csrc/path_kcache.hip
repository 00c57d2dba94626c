// path_kcache: transformed key cache after a prefill of L tokens (gfx950).
//
// The inference form keeps every cached key already carried to "now": after
// token L-1 the cache holds H_{L-1} ... H_{j+1} k_j (Dutch summary section 3,
// "Inferentie"; Chinese notes, inference paragraph).  Per chunk b, path_ut
// gives k~_j = H_{end(b)} ... H_{j+1} k_j.  In row-vector form a chunk c
// acts on a key as
//     k^T <- k^T P_c,   P_c = I - W_c^T Z_c,   Z_c = T_c^{-T} W_c
// (the chunk's UT form), so the cached key is k~_j^T P_{b+1} ... P_{N-1}.
// W_c^T Z_c = M_c^T with M_c = W_c^T T_c^{-1} W_c, the matrix whose I - M_c
// carries the queries through chunk c in the forward: after a bf16 forward
// on the same inputs its workspace holds K~ and -M_c^T for every chunk, and
// path_kcache_from_forward starts from those (the dense form below) instead
// of running path_ut again.
//
// The product of the later chunks is formed by suffix products over groups of
// G = 8 chunks, O(L d^2) work in all (instead of carrying every key through
// every later chunk, O(L^2 d)):
//   1. path_kcache_group_kernel, per (head, group g): every key chunk b of
//      the group carried to the group's end, Y_b = K~_b P_{b+1} ... P_{end(g)}
//      (written over K~), and the group's product T_g = P_{start(g)} ...
//      P_{end(g)}, whose rows are the d identity rows carried through the
//      group (fp32);
//   2. path_kcache_suffix_kernel, per head (and row block of R, d = 128),
//      right to left over the groups: R_{last} = I, R_g = T_{g+1} R_{g+1};
//   3. path_kcache_apply_kernel, per (head, group): K_cache_b = Y_b R_g for
//      the group's chunks.
// V_cache = V is copied by extra workgroups of the suffix launch.
// The carry (step 1) uses the query transport's layout and MFMA orientation
// (the key rides in fp32 accumulators, K^T -= Z^T X^T with X^T = W K^T; -Z^T
// comes from path_ut with its token axis in k-slot order and its d rows
// permuted, so the key's registers hold d in natural order).  In the dense
// form it is K^T += (-M_c) K^T, 2 d^2 flops per key and chunk (the rank-C
// form's 4 C d at d = 2C), with the A operand -M_c read as the transpose of
// the stored -M_c^T tile by LDS transpose loads.  Steps 2 and 3
// keep R_g as R_g^T with permuted rows, Rp[rho][c] = R_g[c][permk(rho)], in
// two bf16 terms (hi, lo): Rp is the A operand of both products, which then
// carry ~16 significant bits, and the output registers again hold d in
// natural order.
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

__device__ __forceinline__ bf16x8 ld8k(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

template <int C, int D, int PITCH, int NT = 256>
__device__ __forceinline__ void stage_rows_k(bf16* dst, const bf16* src, int nvalid, int tid) {
    constexpr int UPR = D / 8;
#pragma unroll
    for (int u = tid; u < C * UPR; u += NT) {
        const int r = u / UPR, d0 = (u % UPR) * 8;
        uint4 val = {0u, 0u, 0u, 0u};
        if (r < nvalid) val = *reinterpret_cast<const uint4*>(src + (size_t)r * D + d0);
        *reinterpret_cast<uint4*>(dst + r * PITCH + d0) = val;
    }
}

template <int ROWS, int COLS, int PITCH, int NT = 256>
__device__ __forceinline__ void stage_tile_k(bf16* dst, const bf16* src, int tid) {
    constexpr int UPR = COLS / 8;
    constexpr int UNITS = ROWS * UPR;
#pragma unroll
    for (int u = tid; u < UNITS; u += NT) {
        const int r = u / UPR, c8 = u % UPR;
        *reinterpret_cast<uint4*>(dst + r * PITCH + c8 * 8) =
            *reinterpret_cast<const uint4*>(src + (size_t)u * 8);
    }
}

}  // namespace

// Step 1.  Workgroup p of group g (8 waves) holds four row chunks of 64
// rows, two waves each: row chunk rc = -D/64 + 4p + (wave >> 1); rc >= 0 is
// the key chunk start(g) + rc, rc < 0 a block of 64 identity rows (entering
// before the group's first chunk).  The workgroup walks the group's chunks
// from the first one any of its row chunks passes; a row chunk is carried
// through those after its own chunk.
template <int D, bool DENSE>
__global__ __launch_bounds__(512, 2) void path_kcache_group_kernel(const KcacheArgs a) {
    constexpr int C = 64, PK = D + 8, PC = C + 8, G = kKcacheGroup, NID = D / 64, NT = 512;
    constexpr int DT = D / 32, KSD = D / 16, KSC = C / 16;
    constexpr int NP = (G + NID + 3) / 4;
    // rank-C form: W rows and Z^T; dense form: the chunk's -M^T as D / 64
    // tiles [D][64] of its columns 64 h .. 64 h + 63 (rows swizzled by swz_v)
    __shared__ __attribute__((aligned(16))) bf16 sW[DENSE ? 8 : C * PK];
    __shared__ __attribute__((aligned(16))) bf16 sZ[DENSE ? 8 : D * PC];
    __shared__ __attribute__((aligned(16))) bf16 sM[DENSE ? D * D : 8];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int L = a.L, N = a.N, Lp = N * C, NG = a.NG;
    const int head = blockIdx.x / (NG * NP);
    const int g = (blockIdx.x / NP) % NG, p = blockIdx.x % NP;
    const int c0 = g * G, c1 = min(c0 + G, N) - 1;
    const int rc = -NID + 4 * p + (wave >> 1);
    const int jloc = (wave & 1) * 32 + l32;
    const int kc = c0 + rc;                       // key chunk (rc >= 0)
    const bool active = rc < 0 || kc <= c1;
    const int start = rc < 0 ? c0 : kc + 1;       // first chunk this row chunk passes
    const int cfirst = c0 + max(-NID + 4 * p + 1, 0);   // first chunk the workgroup needs

    const bf16* kin = static_cast<const bf16*>(a.kt_in) + (size_t)head * Lp * D;   // K~ rows
    bf16* kt = static_cast<bf16*>(a.kt) + (size_t)head * Lp * D;                   // Y rows
    const bf16* win = DENSE ? nullptr : static_cast<const bf16*>(a.w) + (size_t)head * L * D;
    const bf16* zt = DENSE ? nullptr : static_cast<const bf16*>(a.zt) + (size_t)head * N * D * C;
    const bf16* mtg = DENSE ? static_cast<const bf16*>(a.mt) + (size_t)head * N * D * D : nullptr;
    unsigned voff[8];
    if (DENSE) vtr_offsets(voff, lane);

    // register 8s+t of kacc[dt] holds d = 32 dt + 16 s + 8 hh + t; the
    // carried key's bf16 B operand of k-step ks is packed from kacc where it
    // is used (the input rows are bf16, so the first packing is exact)
    f32x16 kacc[DT];
    if (rc >= 0 && active) {
        const bf16* krow = kin + ((size_t)kc * C + jloc) * D;
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
            const bf16x8 k8 = ld8k(krow + 16 * ks + 8 * hh);
#pragma unroll
            for (int t = 0; t < 8; ++t) kacc[ks >> 1][8 * (ks & 1) + t] = static_cast<float>(k8[t]);
        }
    } else {
        const int r = (rc + NID) * C + jloc;      // identity row r
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks)
#pragma unroll
            for (int t = 0; t < 8; ++t) kacc[ks >> 1][8 * (ks & 1) + t] = (16 * ks + 8 * hh + t == r) ? 1.f : 0.f;
    }
    for (int c = cfirst; c <= c1; ++c) {
        __syncthreads();
        if constexpr (DENSE) {
            // every load first, then the stores (the loads' latencies overlap)
            constexpr int UM = D * D / 8 / NT;
            static_assert(UM * NT * 8 == D * D, "whole 16-byte units per thread");
            const bf16* src = mtg + (size_t)c * D * D;
            uint4 m[UM];
#pragma unroll
            for (int i = 0; i < UM; ++i) m[i] = *reinterpret_cast<const uint4*>(src + (size_t)(tid + NT * i) * 8);
#pragma unroll
            for (int i = 0; i < UM; ++i) {
                const int u = tid + NT * i, r = u / (D / 8), cu = u % (D / 8);
                *reinterpret_cast<uint4*>(sM + (cu >> 3) * D * 64 + r * 64 + (((cu & 7) ^ swz_v(r)) << 3)) = m[i];
            }
        } else {
            stage_rows_k<C, D, PK, NT>(sW, win + (size_t)c * C * D, min(C, L - c * C), tid);
            stage_tile_k<D, C, PC, NT>(sZ, zt + (size_t)c * D * C, tid);
        }
        __syncthreads();
        if (!active || c < start) continue;
        if constexpr (DENSE) {
            // K^T += (-M) K^T with the old K^T as the B operand; the A operand
            // A[rho][c] = -M[permk(rho)][c] = mt[permk(c)][permk(rho)] is the
            // transpose of the stored tile (rows rho of the accumulators hold
            // d = permk(rho), i.e. natural d in register order)
            bf16x8 kb[KSD];
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) {
                kb[ks] = pack8k(kacc[ks >> 1], ks & 1);
                // packed here, before the first product overwrites kacc (the
                // compiler would otherwise pack each one at its first use and
                // keep a second copy of the accumulators live until then)
                asm volatile("" : "+v"(kb[ks]));
            }
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) {
                bf16x8 am[DT];
#pragma unroll
                for (int rt = 0; rt < DT; ++rt) am[rt] = pv_operand(sM + (rt >> 1) * D * 64, voff, rt & 1, ks);
#pragma unroll
                for (int rt = 0; rt < DT; ++rt) kacc[rt] = mfma32k(am[rt], kb[ks], kacc[rt]);
                __builtin_amdgcn_sched_barrier(0);      // one k-step's operands live at a time
            }
            continue;
        }
        f32x16 x[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
            for (int v = 0; v < 16; ++v) x[k2][v] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
            const bf16x8 kb = pack8k(kacc[ks >> 1], ks & 1);
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2)
                x[k2] = mfma32k(ld8k(sW + (32 * k2 + l32) * PK + 8 * hh + 16 * ks), kb, x[k2]);
        }
        bf16x8 xB[KSC];
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks) xB[ks] = pack8k(x[ks >> 1], ks & 1);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const bf16* az = sZ + (32 * dt + l32) * PC + 8 * hh;
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) kacc[dt] = mfma32k(ld8k(az + 16 * ks), xB[ks], kacc[dt]);
        }
    }
    if (!active) return;
    if (rc >= 0) {
        // Y_b over K~_b (the key rows are read once, at the start, by their own waves)
        bf16* yrow = kt + ((size_t)kc * C + jloc) * D;
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks)
            *reinterpret_cast<bf16x8*>(yrow + 16 * ks + 8 * hh) = pack8k(kacc[ks >> 1], ks & 1);
    } else {
        // row r of T_g in fp32
        float* trow = a.tg + (((size_t)head * NG + g) * D + (rc + NID) * C + jloc) * D;
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int v = 8 * (ks & 1) + 4 * q;
                *reinterpret_cast<f32x4*>(trow + 16 * ks + 8 * hh + 4 * q) =
                    f32x4{kacc[ks >> 1][v], kacc[ks >> 1][v + 1], kacc[ks >> 1][v + 2], kacc[ks >> 1][v + 3]};
            }
    }
}

// Step 2.  Right to left over the groups, per head.  Rp_g[rho][c] = sum_m
// Rp_{g+1}[rho][m] T_{g+1}[c][m] is R_g[c][permk(rho)]: the A operand
// Rp_{g+1} (two bf16 terms, LDS) times the B operand T_{g+1} rows (fp32,
// split into two bf16 terms), three MFMAs per k-step (hi hi, hi lo, lo hi).
// A row block of Rp_g needs only the same rows of Rp_{g+1}, so the (D/32)^2
// output tiles are split into row blocks over RB workgroups per head, one
// tile per wave: workgroup rb holds rows RPB rb .. +RPB-1, wave w the tile
// i = 4 rb + w (row tile i / (D/32), column tile i % (D/32)).
// workgroups per head of the suffix kernel: one 32 x 32 output tile per wave
constexpr int suffix_blocks(int D) { return (D / 32) * (D / 32) / 4; }
// further workgroups of the suffix launch copy the values into the cache
// while the suffix chains run (those leave most of the chip idle)
constexpr int kValueCopyBlocks = 512;

// V_cache = V for the L prefill slots of every head: workgroup cb of nb, a
// grid-stride loop over rows with D/8 lanes per row (16 bytes each), NF rows
// in flight per lane (the launch's register allocation, sized for the suffix
// products, leaves about one such workgroup per CU: it needs many loads in
// flight to keep up with HBM).
template <int D>
__device__ __forceinline__ void copy_values(const KcacheArgs& a, int cb, int nb) {
    constexpr int UPR = D / 8;                       // 16-byte units per row
    constexpr int RPP = 256 / UPR;                   // rows per workgroup pass
    const int tid = threadIdx.x, unit = tid % UPR;
    const int rows = a.BH * a.L;                     // < 2^31 (checked by the caller's shape limits)
    const int stride = nb * RPP;
    constexpr int NF = 16;
    for (int r0 = cb * RPP + tid / UPR; r0 < rows; r0 += NF * stride) {
        bf16x8 v[NF];
        long long dst[NF];
#pragma unroll
        for (int i = 0; i < NF; ++i) {
            const int r = r0 + i * stride;
            dst[i] = -1;
            if (r < rows) {
                const int head = r / a.L, j = r - head * a.L;
                v[i] = ld8k(static_cast<const bf16*>(a.v) + (size_t)r * D + 8 * unit);
                dst[i] = cache_row(a.map, head, j);
            }
        }
#pragma unroll
        for (int i = 0; i < NF; ++i)
            if (dst[i] >= 0)
                *reinterpret_cast<bf16x8*>(static_cast<bf16*>(a.v_cache) + dst[i] * D + 8 * unit) = v[i];
    }
}

template <int D>
__global__ __launch_bounds__(256) void path_kcache_suffix_kernel(const KcacheArgs a) {
    constexpr int PR = D + 8, CT = D / 32, KSD = D / 16;
    constexpr int RB = suffix_blocks(D);  // workgroups per head
    constexpr int RPB = D / RB;           // Rp rows per workgroup
    __shared__ __attribute__((aligned(16))) bf16 sRh[RPB * PR];
    __shared__ __attribute__((aligned(16))) bf16 sRl[RPB * PR];

    if (static_cast<int>(blockIdx.x) >= a.BH * RB) {  // the value-copy workgroups
        copy_values<D>(a, blockIdx.x - a.BH * RB, gridDim.x - a.BH * RB);
        return;
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int head = blockIdx.x / RB, rb = blockIdx.x % RB, NG = a.NG;
    const int tile = 4 * rb + wave, dt = tile / CT, ct = tile % CT;
    const int r0 = RPB * rb;
    const int c = 32 * ct + l32;
    bf16* rg = static_cast<bf16*>(a.rg) + (size_t)head * NG * 2 * D * D;   // [g][hi, lo][rho][c]

    // R_{NG-1} = I: Rp[rho][c] = (c == permk(rho)), this workgroup's rows
    for (int u = tid; u < RPB * D; u += 256) {
        const int rho = r0 + u / D, cc = u % D;
        const bf16 e = static_cast<bf16>(cc == permk(rho) ? 1.f : 0.f);
        sRh[(rho - r0) * PR + cc] = e;
        sRl[(rho - r0) * PR + cc] = static_cast<bf16>(0.f);
        bf16* out = rg + (size_t)(NG - 1) * 2 * D * D;
        out[rho * D + cc] = e;
        out[D * D + rho * D + cc] = static_cast<bf16>(0.f);
    }
    // B operand: row c of T_{g+1}, k = m = 16 ks + 8 hh .. +7 (fp32), loaded
    // one step ahead
    f32x4 tv[KSD][2];
    auto load_t = [&](int gg) {
        const float* trow = a.tg + (((size_t)head * NG + gg) * D + c) * D;
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks)
#pragma unroll
            for (int q = 0; q < 2; ++q) tv[ks][q] = *reinterpret_cast<const f32x4*>(trow + 16 * ks + 8 * hh + 4 * q);
    };
    if (NG >= 2) load_t(NG - 1);
    const int rl = 32 * dt + l32 - r0;    // the lane's A row in the LDS block
    for (int g = NG - 2; g >= 0; --g) {
        __syncthreads();
        bf16x8 bh[KSD], bl[KSD];
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks)
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float x = tv[ks][t >> 2][t & 3];
                bh[ks][t] = static_cast<bf16>(x);
                bl[ks][t] = static_cast<bf16>(x - static_cast<float>(bh[ks][t]));
            }
        if (g >= 1) load_t(g);
        f32x16 acc;
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
            const bf16x8 ah = ld8k(sRh + rl * PR + 16 * ks + 8 * hh);
            const bf16x8 al = ld8k(sRl + rl * PR + 16 * ks + 8 * hh);
            acc = mfma32k(ah, bh[ks], acc);
            acc = mfma32k(ah, bl[ks], acc);
            acc = mfma32k(al, bh[ks], acc);
        }
        __syncthreads();    // every wave has read Rp_{g+1}
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int rho = 32 * dt + 8 * (v >> 2) + 4 * hh + (v & 3);
            const float x = acc[v];
            const bf16 h = static_cast<bf16>(x);
            sRh[(rho - r0) * PR + c] = h;
            sRl[(rho - r0) * PR + c] = static_cast<bf16>(x - static_cast<float>(h));
        }
        __syncthreads();
        // this workgroup's rows of Rp_g to global memory in 16-byte units
        bf16* out = rg + (size_t)g * 2 * D * D + (size_t)r0 * D;
        for (int u = tid; u < RPB * D / 8; u += 256) {
            const int rho = u / (D / 8), c8 = (u % (D / 8)) * 8;
            *reinterpret_cast<bf16x8*>(out + (size_t)u * 8) = ld8k(sRh + rho * PR + c8);
            *reinterpret_cast<bf16x8*>(out + D * D + (size_t)u * 8) = ld8k(sRl + rho * PR + c8);
        }
    }
}

// Step 3.  One workgroup per (head, group): K_cache^T = Rp_g Y^T for the
// group's chunks (A: Rp_g, hi and lo, in LDS; B: Y rows, exact bf16), one key
// tile of 32 per wave pair and d tiles split between the pair (the values
// are copied by the suffix launch).
template <int D>
__global__ __launch_bounds__(256, 2) void path_kcache_apply_kernel(const KcacheArgs a) {
    constexpr int C = 64, PR = D + 8, DT = D / 32, KSD = D / 16, DTW = DT / 2;
    __shared__ __attribute__((aligned(16))) bf16 sRh[D * PR];
    __shared__ __attribute__((aligned(16))) bf16 sRl[D * PR];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int L = a.L, N = a.N, Lp = N * C, NG = a.NG;
    const int head = blockIdx.x / NG, g = blockIdx.x % NG;
    const int c0 = g * kKcacheGroup, c1 = min(c0 + kKcacheGroup, N) - 1;
    const bf16* rg = static_cast<const bf16*>(a.rg) + ((size_t)head * NG + g) * 2 * D * D;
    for (int u = tid; u < D * D / 8; u += 256) {
        const int rho = u / (D / 8), c8 = (u % (D / 8)) * 8;
        *reinterpret_cast<bf16x8*>(sRh + rho * PR + c8) = ld8k(rg + (size_t)u * 8);
        *reinterpret_cast<bf16x8*>(sRl + rho * PR + c8) = ld8k(rg + D * D + (size_t)u * 8);
    }
    __syncthreads();
    const bf16* kt = static_cast<const bf16*>(a.kt) + (size_t)head * Lp * D;
    const int jloc = (wave & 1) * 32 + l32, dtb = (wave >> 1) * DTW;
    const int cend = min(c1, (L - 1) / C);        // chunks past it are padding
    // Y rows as the B operand (k = c = 16 ks + 8 hh .. +7), one chunk ahead
    bf16x8 ynext[KSD];
    auto load_y = [&](int b) {
        const bf16* yrow = kt + ((size_t)b * C + jloc) * D;
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) ynext[ks] = ld8k(yrow + 16 * ks + 8 * hh);
    };
    if (c0 <= cend) load_y(c0);
    for (int b = c0; b <= cend; ++b) {            // uniform: every lane runs the MFMAs
        const int j = b * C + jloc;
        bf16x8 y8[KSD];
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) y8[ks] = ynext[ks];
        if (b < cend) load_y(b + 1);
        f32x16 acc[DTW];
#pragma unroll
        for (int i = 0; i < DTW; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
#pragma unroll
            for (int i = 0; i < DTW; ++i) {
                const int rho = 32 * (dtb + i) + l32;
                acc[i] = mfma32k(ld8k(sRh + rho * PR + 16 * ks + 8 * hh), y8[ks], acc[i]);
                acc[i] = mfma32k(ld8k(sRl + rho * PR + 16 * ks + 8 * hh), y8[ks], acc[i]);
            }
        }
        if (j >= L) continue;                     // padding rows of the last chunk
        const long long row = cache_row(a.map, head, j);
        if (row < 0) continue;
        // register 8s+t of tile dt holds d = 32 dt + 16 s + 8 hh + t
        bf16* kout = static_cast<bf16*>(a.k_cache) + row * D;
#pragma unroll
        for (int i = 0; i < DTW; ++i)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
                *reinterpret_cast<bf16x8*>(kout + 32 * (dtb + i) + 16 * s2 + 8 * hh) = pack8k(acc[i], s2);
    }
}

hipError_t launch_path_kcache(const KcacheArgs& a, int D, hipStream_t s) {
    const int NG = a.NG;
    const bool dense = a.mt != nullptr;
    if (D == 64) {
        constexpr int NP = (kKcacheGroup + 1 + 3) / 4;
        if (dense) hipLaunchKernelGGL((path_kcache_group_kernel<64, true>), dim3(a.BH * NG * NP), dim3(512), 0, s, a);
        else hipLaunchKernelGGL((path_kcache_group_kernel<64, false>), dim3(a.BH * NG * NP), dim3(512), 0, s, a);
        hipLaunchKernelGGL(path_kcache_suffix_kernel<64>, dim3(a.BH * suffix_blocks(64) + kValueCopyBlocks), dim3(256), 0, s, a);
        hipLaunchKernelGGL(path_kcache_apply_kernel<64>, dim3(a.BH * NG), dim3(256), 0, s, a);
    } else if (D == 128) {
        constexpr int NP = (kKcacheGroup + 2 + 3) / 4;
        if (dense) hipLaunchKernelGGL((path_kcache_group_kernel<128, true>), dim3(a.BH * NG * NP), dim3(512), 0, s, a);
        else hipLaunchKernelGGL((path_kcache_group_kernel<128, false>), dim3(a.BH * NG * NP), dim3(512), 0, s, a);
        hipLaunchKernelGGL(path_kcache_suffix_kernel<128>, dim3(a.BH * suffix_blocks(128) + kValueCopyBlocks), dim3(256), 0, s, a);
        hipLaunchKernelGGL(path_kcache_apply_kernel<128>, dim3(a.BH * NG), dim3(256), 0, s, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace path
