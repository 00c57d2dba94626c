// path_fwd (bf16 mode): blockwise PaTH attention forward on gfx950 MFMA.
//
// Algorithm (Dutch summary section 3: boundary-adjusted queries/keys per
// block, a right-to-left scan over key/value blocks, FlashAttention-style
// on-chip tiling; Chinese notes, training strategy: UT transform and the
// full-matrix form).  Chunks hold C = 64 tokens.  A wave owns 32 queries of
// one chunk a and walks the key chunks b = a, a-1, ..., 0:
//   b = a:  S = Q K~^T + strictUpper(Q W^T) Y   (causal mask j <= i)
//           Q <- Q - lower(Q W^T) U             (query carried to chunk start)
//   b < a:  S = Q K~^T,  X = Q W^T
//           Q <- Q - X U   (skipped for b = 0)  (query carried through chunk b)
// and accumulates softmax(S) V online.  Every product is a bf16 MFMA with
// fp32 accumulation; the carried query Q stays in fp32 accumulators and is
// rounded to bf16 only as an MFMA operand.
//
// Orientation.  All products are formed transposed (S^T = K~ Q^T,
// X^T = W Q^T, O^T += V^T P^T, Q^T -= U^T X^T), so every accumulator that
// feeds a later product (S^T -> P^T, X^T, Q^T) is already in B-operand
// position: accumulator registers 8s..8s+7 are the B operand of k-step s,
// under the k-slot permutation perm16 (see path_internal.h).  The A operands
// (K~, W along d; V^T, U^T, Y^T along keys) sit in LDS with that permutation
// applied, so they are plain 16-byte LDS reads: K~, U^T and Y^T are written
// pre-permuted by path_ut; W is permuted (groups of four d) and V transposed
// while they are staged from the inputs.
//
// Workgroup: 4 waves = 128 queries = query chunks 2qb and 2qb+1.  Key chunks
// are staged once per workgroup in LDS and shared by the 4 waves.  Block
// order: heaviest query blocks first; when BH is a multiple of 8 all blocks
// of one head land on one XCD (blocks are dealt to the 8 XCDs round-robin),
// so a head's K~/W/U/V chunks are reused out of that XCD's L2.
#include "path_internal.h"

namespace path {

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// accumulator registers 8*half .. 8*half+7 as a bf16 B operand
__device__ __forceinline__ bf16x8 pack8(const f32x16& acc, int half) {
    bf16x8 r;
#pragma unroll
    for (int t = 0; t < 8; ++t) r[t] = static_cast<bf16>(acc[8 * half + t]);
    return r;
}

__device__ __forceinline__ bf16x8 lds8(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}

// copy a [rows][cols] bf16 tile (contiguous in global) to LDS with row pitch
template <int ROWS, int COLS, int PITCH>
__device__ __forceinline__ void stage_tile(bf16* dst, const bf16* src, int tid) {
    constexpr int UPR = COLS / 8;              // 16-byte units per row
    constexpr int UNITS = ROWS * UPR;
#pragma unroll
    for (int u = tid; u < UNITS; u += 256) {
        const int r = u / UPR, c8 = u % UPR;
        const uint4 val = *reinterpret_cast<const uint4*>(src + (size_t)u * 8);
        *reinterpret_cast<uint4*>(dst + r * PITCH + c8 * 8) = val;
    }
}

// W rows [C][D] (input, rows >= nvalid are padding) -> LDS [C][PITCH] with
// the d axis permuted: d-quad q of each group of 16 goes to slot quad perm(q)
template <int C, int D, int PITCH>
__device__ __forceinline__ void stage_w_perm(bf16* dst, const bf16* src, int nvalid, int tid) {
    constexpr int UPR = D / 8;
#pragma unroll
    for (int u = tid; u < C * UPR; u += 256) {
        const int r = u / UPR, d0 = (u % UPR) * 8;
        uint4 val = {0u, 0u, 0u, 0u};
        if (r < nvalid) val = *reinterpret_cast<const uint4*>(src + (size_t)r * D + d0);
        const int s0 = permk(d0), s1 = permk(d0 + 4);
        *reinterpret_cast<uint2*>(dst + r * PITCH + s0) = make_uint2(val.x, val.y);
        *reinterpret_cast<uint2*>(dst + r * PITCH + s1) = make_uint2(val.z, val.w);
    }
}

// V rows [C][D] (input) -> LDS V^T [D][PITCH] with the key axis permuted.
// Each work item moves a quad of keys x 8 values of d.
template <int C, int D, int PITCH>
__device__ __forceinline__ void stage_v_trans(bf16* dst, const bf16* src, int nvalid, int tid) {
    constexpr int ITEMS = (C / 4) * (D / 8);
#pragma unroll
    for (int it = tid; it < ITEMS; it += 256) {
        const int kq = it / (D / 8), d0 = (it % (D / 8)) * 8;
        bf16x8 rows[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = 4 * kq + r;
            rows[r] = bf16x8{};
            if (j < nvalid) rows[r] = *reinterpret_cast<const bf16x8*>(src + (size_t)j * D + d0);
        }
        const int slot = permk(4 * kq);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            bf16x4 col = {rows[0][e], rows[1][e], rows[2][e], rows[3][e]};
            *reinterpret_cast<bf16x4*>(dst + (d0 + e) * PITCH + slot) = col;
        }
    }
}

__device__ __forceinline__ void decode_block(int bid, int BH, int nqb, int& head, int& qb) {
    if ((BH & 7) == 0) {
        const int xcd = bid & 7, j = bid >> 3;
        head = xcd + 8 * (j / nqb);
        qb = nqb - 1 - (j % nqb);
    } else {
        head = bid / nqb;
        qb = nqb - 1 - (bid % nqb);
    }
}

template <int D, bool GATE>
__global__ __launch_bounds__(256, (D == 64 ? 2 : 1)) void path_fwd_bf16_kernel(const FwdArgs a) {
    constexpr int C = 64;
    constexpr int PK = D + 8;     // pitch of [key][d] tiles
    constexpr int PC = C + 8;     // pitch of [d][key] and [key][key] tiles
    constexpr int DT = D / 32;    // 32-row tiles along d
    constexpr int KSD = D / 16;   // k-steps along d
    constexpr int KSC = C / 16;   // k-steps along keys (4)

    __shared__ __attribute__((aligned(16))) bf16 sK[C * PK];
    __shared__ __attribute__((aligned(16))) bf16 sW[C * PK];
    __shared__ __attribute__((aligned(16))) bf16 sU[D * PC];
    __shared__ __attribute__((aligned(16))) bf16 sV[D * PC];
    __shared__ __attribute__((aligned(16))) bf16 sY[C * PC];
    __shared__ __attribute__((aligned(16))) float sLoc[C];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const int L = a.L, N = a.N, Lp = N * C;
    int head, qb;
    decode_block(blockIdx.x, a.BH, a.nqb, head, qb);

    const int qc = 2 * qb + (wave >> 1);      // this wave's query chunk
    const bool active = qc < N;
    const int iloc = (wave & 1) * 32 + l32;   // query row within its chunk
    const int qi = qc * C + iloc;
    const bool qvalid = active && qi < L;

    const bf16* qrow = static_cast<const bf16*>(a.q) + ((size_t)head * L + (qvalid ? qi : 0)) * D;
    const bf16* kt = static_cast<const bf16*>(a.kt) + (size_t)head * Lp * D;
    const bf16* win = static_cast<const bf16*>(a.w) + (size_t)head * L * D;
    const bf16* vin = static_cast<const bf16*>(a.v) + (size_t)head * L * D;
    const bf16* ut = static_cast<const bf16*>(a.ut) + (size_t)head * N * D * C;
    const bf16* yt = static_cast<const bf16*>(a.yt) + (size_t)head * N * C * C;

    // carried query (fp32, accumulator layout) and its bf16 B operand
    f32x16 qacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            bf16x4 q4 = {};
            if (qvalid) q4 = *reinterpret_cast<const bf16x4*>(qrow + 32 * dt + 8 * r4 + 4 * hh);
#pragma unroll
            for (int t = 0; t < 4; ++t) qacc[dt][4 * r4 + t] = static_cast<float>(q4[t]);
        }
    bf16x8 qB[KSD];
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) qB[ks] = pack8(qacc[ks >> 1], ks & 1);

    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[dt][v] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    float loc_i = 0.f;
    double dab = 0.0;
    if (GATE && qvalid) loc_i = a.loc[(size_t)head * Lp + qi];
    const float c2 = a.scale2;

    const int top = min(2 * qb + 1, N - 1);
    for (int kc = top; kc >= 0; --kc) {
        __syncthreads();
        const int nvalid = min(C, L - kc * C);
        stage_tile<C, D, PK>(sK, kt + (size_t)kc * C * D, tid);
        stage_w_perm<C, D, PK>(sW, win + (size_t)kc * C * D, nvalid, tid);
        stage_tile<D, C, PC>(sU, ut + (size_t)kc * D * C, tid);
        stage_v_trans<C, D, PC>(sV, vin + (size_t)kc * C * D, nvalid, tid);
        if (kc >= 2 * qb) stage_tile<C, C, PC>(sY, yt + (size_t)kc * C * C, tid);
        if (GATE && tid < C) sLoc[tid] = a.loc[(size_t)head * Lp + kc * C + tid];
        __syncthreads();
        if (!active || kc > qc) continue;
        const bool diag = (kc == qc);

        // S^T = K~ Q^T and X^T = W Q^T  (2 tiles of 32 keys)
        f32x16 s[2], x[2];
#pragma unroll
        for (int kt2 = 0; kt2 < 2; ++kt2) {
#pragma unroll
            for (int v = 0; v < 16; ++v) { s[kt2][v] = 0.f; x[kt2][v] = 0.f; }
            const bf16* ak = sK + (32 * kt2 + l32) * PK + 8 * hh;
            const bf16* aw = sW + (32 * kt2 + l32) * PK + 8 * hh;
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) {
                s[kt2] = mfma32(lds8(ak + 16 * ks), qB[ks], s[kt2]);
                x[kt2] = mfma32(lds8(aw + 16 * ks), qB[ks], x[kt2]);
            }
        }
        if (diag) {
            // S^T += Y^T strictUpper(X)^T ; X^T <- lower part (m <= i)
            bf16x8 xu[KSC];
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks)
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int v = 8 * (ks & 1) + t;
                    const int m = 32 * (ks >> 1) + 8 * (v >> 2) + 4 * hh + (v & 3);
                    const float xv = x[ks >> 1][v];
                    xu[ks][t] = static_cast<bf16>(m > iloc ? xv : 0.f);
                    x[ks >> 1][v] = (m <= iloc) ? xv : 0.f;
                }
#pragma unroll
            for (int kt2 = 0; kt2 < 2; ++kt2) {
                const bf16* ay = sY + (32 * kt2 + l32) * PC + 8 * hh;
#pragma unroll
                for (int ks = 0; ks < KSC; ++ks) s[kt2] = mfma32(lds8(ay + 16 * ks), xu[ks], s[kt2]);
            }
        }

        // online softmax (log2 units).  Lane holds keys
        // j = 32*kt2 + 8*(v/4) + 4*hh + v%4 of query iloc; lane^32 holds the rest.
        const float a_i = GATE ? loc_i + static_cast<float>(dab) : 0.f;
        float mx = -INFINITY;
#pragma unroll
        for (int kt2 = 0; kt2 < 2; ++kt2)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                f32x4 lj = {0.f, 0.f, 0.f, 0.f};
                if (GATE) lj = *reinterpret_cast<const f32x4*>(sLoc + 32 * kt2 + 8 * r4 + 4 * hh);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int v = 4 * r4 + t;
                    const int j = 32 * kt2 + 8 * r4 + 4 * hh + t;
                    float z = GATE ? fmaf(s[kt2][v], c2, -lj[t]) : s[kt2][v];
                    if (diag && j > iloc) z = -INFINITY;
                    s[kt2][v] = z;
                    mx = fmaxf(mx, z);
                }
            }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = GATE ? fmaxf(m_run, mx + a_i) : fmaxf(m_run, mx * c2);
        const float alpha = exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int v = 0; v < 16; ++v) oacc[dt][v] *= alpha;
        const float msub = GATE ? m_new - a_i : m_new;
        bf16x8 pB[KSC];
        float psum = 0.f;
#pragma unroll
        for (int ks = 0; ks < KSC; ++ks)
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float z = s[ks >> 1][8 * (ks & 1) + t];
                const float p = GATE ? exp2f(z - msub) : exp2f(fmaf(z, c2, -msub));
                psum += p;
                pB[ks][t] = static_cast<bf16>(p);
            }
        l_run += psum;

        // O^T += V^T P^T
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const bf16* av = sV + (32 * dt + l32) * PC + 8 * hh;
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) oacc[dt] = mfma32(lds8(av + 16 * ks), pB[ks], oacc[dt]);
        }
        // carry the query through chunk kc:  Q^T += (-U^T) X^T
        if (kc > 0) {
            bf16x8 xB[KSC];
#pragma unroll
            for (int ks = 0; ks < KSC; ++ks) xB[ks] = pack8(x[ks >> 1], ks & 1);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const bf16* au = sU + (32 * dt + l32) * PC + 8 * hh;
#pragma unroll
                for (int ks = 0; ks < KSC; ++ks) qacc[dt] = mfma32(lds8(au + 16 * ks), xB[ks], qacc[dt]);
            }
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) qB[ks] = pack8(qacc[ks >> 1], ks & 1);
            if (GATE) dab += static_cast<double>(a.csum[(size_t)head * N + kc]);
        }
    }

    if (!active) return;
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (!qvalid) return;
    const float inv = 1.f / l_tot;
    bf16* orow = static_cast<bf16*>(a.out) + ((size_t)head * L + qi) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            bf16x4 o4;
#pragma unroll
            for (int t = 0; t < 4; ++t) o4[t] = static_cast<bf16>(oacc[dt][4 * r4 + t] * inv);
            *reinterpret_cast<bf16x4*>(orow + 32 * dt + 8 * r4 + 4 * hh) = o4;
        }
    if (a.lse && hh == 0) a.lse[(size_t)head * L + qi] = (m_run + log2f(l_tot)) * kLn2;
}

hipError_t launch_path_fwd_bf16(const FwdArgs& a, bool gate, hipStream_t s) {
    const dim3 grid(a.BH * a.nqb), block(256);
    if (a.D == 64) {
        if (gate) hipLaunchKernelGGL((path_fwd_bf16_kernel<64, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((path_fwd_bf16_kernel<64, false>), grid, block, 0, s, a);
    } else if (a.D == 128) {
        if (gate) hipLaunchKernelGGL((path_fwd_bf16_kernel<128, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((path_fwd_bf16_kernel<128, false>), grid, block, 0, s, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace path
