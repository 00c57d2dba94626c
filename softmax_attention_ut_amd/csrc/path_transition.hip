// Transition parameters of every token from the layer input (Chinese notes,
// "key design"; Dutch summary section 2, "Kernmechanisme"):
//     z_t = W_up (W_down x_t),  c_t = conv0 * z_t + conv1 * z_{t-1} + conv2 * z_{t-2},
//     w_t = per-head L2 normalisation of c_t,  beta_t = 2 sigmoid(u . x_t + b).
//
// One 256-thread workgroup per tile of 64 consecutive tokens of one sequence
// (so the 4K-token workload is one round of two workgroups per CU).  The two
// tokens before the tile, which the convolution reaches, are recomputed as a
// fifth, mostly empty MFMA token tile (the "halo"), so every token's w
// depends only on its own workgroup.
//
// Stage 1 (every element of x is read once from HBM; every workgroup reads
// the whole of [W_down; u] from L2, which costs more than the x reads):
//     [W_down; u] (r + H channels) x x^T on 16x16x32 bf16 MFMA, fp32
//     accumulators.  x is staged in LDS 128 columns at a time (double
//     buffered, one barrier per stage) and read as the B operand by all four
//     waves; wave q computes channel tiles q and q + 4 for all 64 (+2) tokens,
//     with its weight rows read from global memory.  Channels < r are
//     y = W_down x; the rest give beta.  y goes to LDS as a bf16 (high, low)
//     pair.  x is copied two steps ahead of its use, the weights one step
//     ahead.
// Stage 2 (per head, one wave per head):
//     W_up[head] x y^T on MFMA (high and low parts of y), so a lane holds one
//     token and four consecutive channels.  The four token tiles interleave
//     the tokens (tile tt holds tokens 4 j + tt of lane column j), so the
//     convolution's tokens one and two back are mostly in the same lane; the
//     rest come through one DPP row shift per four values, with the halo
//     entering at lane 0.  The squared norm is summed over the lane's
//     channels and across the four lane groups, and the normalised bf16 rows
//     are staged in LDS and written as whole 16-byte units.
#include "path_attn.h"
#include "path_internal.h"

namespace path {

namespace {

constexpr int kTok = 64;               // tokens per workgroup
constexpr int kHalo = 2;               // the convolution reaches two tokens back
constexpr int kRows = kTok + kHalo;    // staged rows: the tile, then tokens t0-1, t0-2
constexpr int kKc = 128;               // x columns staged per step

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ bf16x8 zero8() {
    bf16x8 z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = static_cast<bf16>(0.f);
    return z;
}

// DPP controls (within each row of 16 lanes)
constexpr int kRowShl = 0x100;   // + n: lane j reads lane j + n (j > 15 - n: invalid)
constexpr int kRowShr = 0x110;   // + n: lane j reads lane j - n (j < n: invalid)

// lane j > 0 of each row of 16 lanes gets v from lane j - 1; lane 0 keeps `old`
__device__ __forceinline__ float row_shr1(float v, float old) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        __builtin_bit_cast(int, old), __builtin_bit_cast(int, v), kRowShr + 1, 0xf, 0xf, false));
}
// lane j < 15 of each row gets v from lane j + 1 (lane 15 gets 0)
__device__ __forceinline__ float row_shl1(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v),
                                                              kRowShl + 1, 0xf, 0xf, true));
}

template <int D, int R>
__global__ __launch_bounds__(256, 2) void path_transition_kernel(const TransArgs a) {
    constexpr int XROW = kKc * 2;                  // bytes per staged x row
    constexpr int XBUF = kRows * XROW;             // one x stage
    constexpr int YROW = 2 * R + 16;               // bytes per y row (padded)
    constexpr int SROW = 2 * D + 16;               // bytes per output staging row
    constexpr int SBUF = kTok * SROW;              // one wave's output staging
    constexpr int REGION = (2 * XBUF > 4 * SBUF) ? 2 * XBUF : 4 * SBUF;
    constexpr int KS = R / 32;                     // k-steps of the second product
    constexpr int CT = D / 16;                     // channel tiles of a head
    __shared__ __align__(16) char lds[REGION + 2 * kRows * YROW];
    char* const xs = lds;                          // x stages, later the output staging
    char* const yhi = lds + REGION;
    char* const ylo = yhi + kRows * YROW;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform (scalar)
    const int col = lane & 15, grp = lane >> 4;
    const int seq = blockIdx.x / a.ntile, tile = blockIdx.x % a.ntile;
    const int t0 = tile * kTok;                    // token of local row 0
    const int L = a.L, Dm = a.Dm, H = a.H;
    const bf16* const x = static_cast<const bf16*>(a.x) + (size_t)seq * L * Dm;

    // ---- stage 1: [W_down; u] x^T ---------------------------------------
    // x copy: 64 rows x 16 units of 16 bytes per stage, 4 units per thread,
    // and a fifth unit for the halo rows 64 + m = token t0 - 1 - m (m = 0, 1;
    // the four waves copy the same 32 units); unit un of row rr is stored at
    // unit un ^ (rr & 15) (conflict-free reads)
    // Loads are never branched around (rows outside the sequence read a
    // clamped row and are zeroed after the load), so the compiler can count
    // the copies in flight instead of waiting for all of them.
    auto xrow = [&](int i) { return i < 4 ? (tid + 256 * i) >> 4 : kTok + ((tid >> 4) & 1); };
    auto xtok = [&](int rr) { return rr < kTok ? t0 + rr : t0 - 1 - (rr - kTok); };
    auto load_x = [&](bf16x8 (&pre)[5], int k0) {
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int rr = xrow(i), un = tid & 15, t = xtok(rr);
            const bf16x8 v = ld8(x + (size_t)min(max(t, 0), L - 1) * Dm + k0 + 8 * un);
            pre[i] = (t >= 0 && t < L) ? v : zero8();
        }
    };
    auto store_x = [&](const bf16x8 (&pre)[5], int buf) {
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int rr = xrow(i), un = tid & 15;
            *reinterpret_cast<bf16x8*>(xs + buf * XBUF + rr * XROW + ((un ^ (rr & 15)) << 4)) =
                pre[i];
        }
    };

    // this wave's channel tiles q and q + 4: lane row = channel 16 * tile + col
    // (channels past r + H read row col of W_down and are zeroed)
    const int nch = R + H;
    const bf16* src[2];
    bool live[2], real[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int ct = wave + 4 * c, ch = 16 * ct + col;
        live[c] = 16 * ct < nch;                   // wave-uniform
        real[c] = ch < nch;
        src[c] = ch < R ? static_cast<const bf16*>(a.w_down) + (size_t)ch * Dm
               : ch < nch ? static_cast<const bf16*>(a.u) + (size_t)(ch - R) * Dm
               : static_cast<const bf16*>(a.w_down) + (size_t)(col % R) * Dm;
    }
    auto load_w = [&](bf16x8 (&wa)[2][4], int k0) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 v = ld8(src[c] + k0 + 32 * ks + 8 * grp);
                wa[c][ks] = real[c] ? v : zero8();
            }
    };

    // token tiles 0-3: local tokens 16 tt + col; tile 4 (halo): column
    // col < 2 is token t0 - 1 - col, the other columns are zero
    f32x4 acc[2][5];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int tt = 0; tt < 5; ++tt) acc[c][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // x chunks are copied two steps ahead: while chunk kc is multiplied from
    // LDS, chunk kc + 1 is in flight in one register set and chunk kc + 2 is
    // issued into the other; the weights (L2) are loaded one step ahead into
    // the other of two register sets (no register copies, which would wait
    // for the newest loads)
    const int nk = Dm / kKc;
    bf16x8 wa[2][4], wb[2][4], xa[5], xb[5];
    load_x(xa, 0);
    load_w(wa, 0);
    load_x(xb, min(1, nk - 1) * kKc);
    store_x(xa, 0);
    __syncthreads();
    auto step = [&](int kc, const bf16x8 (&inflight)[5], bf16x8 (&freeset)[5],
                    const bf16x8 (&wcur)[2][4], bf16x8 (&wnext)[2][4]) {
        // past the last chunk the copies re-read the last one (never used)
        load_x(freeset, min(kc + 2, nk - 1) * kKc);
        load_w(wnext, min(kc + 1, nk - 1) * kKc);
        __builtin_amdgcn_sched_barrier(0);
        const char* xbuf = xs + (kc & 1) * XBUF;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x8 xv[5];
#pragma unroll
            for (int tt = 0; tt < 5; ++tt) {
                const int rr = tt < 4 ? 16 * tt + col : kTok + (col & 1);
                xv[tt] = *reinterpret_cast<const bf16x8*>(xbuf + rr * XROW +
                                                          (((4 * ks + grp) ^ (rr & 15)) << 4));
            }
            if (col >= kHalo) xv[4] = zero8();
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                if (!live[c]) continue;
#pragma unroll
                for (int tt = 0; tt < 5; ++tt) acc[c][tt] = mfma16(wcur[c][ks], xv[tt], acc[c][tt]);
            }
        }
        if (kc + 1 < nk) store_x(inflight, (kc + 1) & 1);
        __syncthreads();
    };
    for (int kc = 0; kc < nk; kc += 2) {
        step(kc, xb, xa, wa, wb);
        if (kc + 1 < nk) step(kc + 1, xa, xb, wb, wa);
    }

    // accumulator (c, tt) register i: channel 16 * (wave + 4c) + 4 grp + i, local token 16 tt + col
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int ct = wave + 4 * c;
        if (!live[c]) continue;
        if (16 * ct < R) {
#pragma unroll
            for (int tt = 0; tt < 5; ++tt) {
                bf16x4 hi, lo;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float v = acc[c][tt][i];
                    hi[i] = static_cast<bf16>(v);
                    lo[i] = static_cast<bf16>(v - static_cast<float>(hi[i]));
                }
                if (tt == 4 && col >= kHalo) continue;
                const int rr = tt < 4 ? 16 * tt + col : kTok + col;
                const int off = rr * YROW + (16 * ct + 4 * grp) * 2;
                *reinterpret_cast<bf16x4*>(yhi + off) = hi;
                *reinterpret_cast<bf16x4*>(ylo + off) = lo;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int h = 16 * ct + 4 * grp + i - R;
                if (h >= H) continue;
                const float bh = a.b[h];
                float* const bout = a.beta + ((size_t)seq * H + h) * L;
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const int t = t0 + 16 * tt + col;
                    if (t < L)
                        bout[t] = 2.f / (1.f + expf(-(acc[c][tt][i] + bh)));
                }
            }
        }
    }
    __syncthreads();

    // ---- stage 2: per head, W_up[head] y^T, convolution, norm ------------
    // Token tile tt of this stage holds the local tokens 4 j + tt (j = lane
    // column), so tokens one and two back are in the same lane except for
    // tile 0 (tiles 3 and 2 of the column before) and tile 1 (tile 3 of the
    // column before): one lane shift per four values.  Column 0 has no column
    // before: its tokens -1 and -2 come from the halo tile (columns 0 and 1).
    bf16x8 yb[4][KS][2];                           // the same B operands for every head
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int off = (4 * col + tt) * YROW + (32 * ks + 8 * grp) * 2;
            yb[tt][ks][0] = *reinterpret_cast<const bf16x8*>(yhi + off);
            yb[tt][ks][1] = *reinterpret_cast<const bf16x8*>(ylo + off);
        }

    char* const stg = xs + wave * SBUF;
    const bf16* const wup = static_cast<const bf16*>(a.w_up);
    const int nrows = min(kTok, L - t0);           // tokens of this tile that exist

    // Each step's W_up rows and convolution taps are loaded one step ahead.
    struct Par {
        bf16x8 wu[KS];
        float tap[4][3];
    };
    auto load_par = [&](int h, int ct2, Par& p) {
        const int e = h * D + 16 * ct2;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            p.wu[ks] = ld8(wup + (size_t)(e + col) * R + 32 * ks + 8 * grp);
        const float* const cp = a.conv + (size_t)(e + 4 * grp) * 3;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int k = 0; k < 3; ++k) p.tap[i][k] = cp[3 * i + k];
    };
    // convolved channels 16 ct2 + 4 grp + i of local tokens 4 col + tt
    auto conv_tile = [&](const Par& p, f32x4 (&cv)[4]) {
        f32x4 z[4], zh = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            z[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                z[tt] = mfma16(p.wu[ks], yb[tt][ks][0], z[tt]);
                z[tt] = mfma16(p.wu[ks], yb[tt][ks][1], z[tt]);
            }
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            // halo operands, read from LDS per tile (registers are short)
            const int off = (kTok + (col & 1)) * YROW + (32 * ks + 8 * grp) * 2;
            const bf16x8 hh = *reinterpret_cast<const bf16x8*>(yhi + off);
            const bf16x8 hl = *reinterpret_cast<const bf16x8*>(ylo + off);
            zh = mfma16(p.wu[ks], col < kHalo ? hh : zero8(), zh);
            zh = mfma16(p.wu[ks], col < kHalo ? hl : zero8(), zh);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // lane 0 of each row: token -1 is halo column 0, token -2 column 1
            const float b3 = row_shr1(z[3][i], zh[i]);
            const float b2 = row_shr1(z[2][i], row_shl1(zh[i]));
            const float t0_ = p.tap[i][0], t1_ = p.tap[i][1], t2_ = p.tap[i][2];
            cv[0][i] = t0_ * z[0][i] + t1_ * b3 + t2_ * b2;
            cv[1][i] = t0_ * z[1][i] + t1_ * z[0][i] + t2_ * b3;
            cv[2][i] = t0_ * z[2][i] + t1_ * z[1][i] + t2_ * z[0][i];
            cv[3][i] = t0_ * z[3][i] + t1_ * z[2][i] + t2_ * z[1][i];
        }
    };

    // the normalised rows of head h: staged in LDS, then written as whole
    // 16-byte units (rows 0 .. nrows - 1 are one contiguous run)
    auto write_head = [&](int h) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        bf16* const wout = static_cast<bf16*>(a.w) + (((size_t)seq * H + h) * L + t0) * D;
        const int units = nrows * (D / 8);
        for (int u = lane; u < units; u += 64) {
            const int rr = u / (D / 8), un = u % (D / 8);
            *reinterpret_cast<bf16x8*>(wout + (size_t)u * 8) =
                *reinterpret_cast<const bf16x8*>(stg + rr * SROW + un * 16);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    auto stage_rows = [&](int ct2, const f32x4 (&cv)[4], const float (&inv)[4]) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            bf16x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = static_cast<bf16>(cv[tt][i] * inv[tt]);
            *reinterpret_cast<bf16x4*>(stg + (4 * col + tt) * SROW + (16 * ct2 + 4 * grp) * 2) = o;
        }
    };
    auto add_sq = [&](const f32x4 (&cv)[4], float (&ss)[4]) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) ss[tt] += cv[tt][i] * cv[tt][i];
    };
    // 1 / norm of each token's d channels: the lane's own sum, then across
    // the four lane groups that hold the other channels of the same token
    auto inv_norm = [&](const float (&ss)[4], float (&inv)[4]) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            float s2 = ss[tt];
            s2 += __shfl_xor(s2, 16);
            s2 += __shfl_xor(s2, 32);
            inv[tt] = s2 > 0.f ? 1.f / sqrtf(s2) : 0.f;
        }
    };

    const int nh = (H - wave + 3) / 4;             // heads of this wave: wave + 4 hi
    Par cur, nxt;
    if (nh > 0) load_par(wave, 0, nxt);
    if constexpr (CT <= 4) {
        // d = 64: a head's channels stay in registers until its norm is known
        for (int hi = 0; hi < nh; ++hi) {
            const int h = wave + 4 * hi;
            f32x4 keep[CT][4];
            float ss[4] = {0.f, 0.f, 0.f, 0.f}, inv[4];
#pragma unroll
            for (int ct2 = 0; ct2 < CT; ++ct2) {
                cur = nxt;
                // the next step's parameters (after the last head: its own again)
                if (ct2 + 1 < CT) load_par(h, ct2 + 1, nxt);
                else load_par(hi + 1 < nh ? h + 4 : h, 0, nxt);
                __builtin_amdgcn_sched_barrier(0);
                conv_tile(cur, keep[ct2]);
                add_sq(keep[ct2], ss);
            }
            inv_norm(ss, inv);
#pragma unroll
            for (int ct2 = 0; ct2 < CT; ++ct2) stage_rows(ct2, keep[ct2], inv);
            write_head(h);
        }
    } else {
        // d = 128: each channel tile is computed twice, first for the norm,
        // then for the values (keeping all of them live would spill).  Step q:
        // head wave + 4 (q / 2CT), pass (q / CT) % 2, channel tile q % CT.
        const int nq = nh * 2 * CT;
        float ss[4], inv[4];
        for (int q = 0; q < nq; ++q) {
            cur = nxt;
            const int qn = min(q + 1, nq - 1);
            load_par(wave + 4 * (qn / (2 * CT)), qn % CT, nxt);
            __builtin_amdgcn_sched_barrier(0);
            const int h = wave + 4 * (q / (2 * CT)), ct2 = q % CT;
            f32x4 cv[4];
            conv_tile(cur, cv);
            if (((q / CT) & 1) == 0) {
                if (ct2 == 0) {
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) ss[tt] = 0.f;
                }
                add_sq(cv, ss);
                if (ct2 == CT - 1) inv_norm(ss, inv);
                continue;
            }
            stage_rows(ct2, cv, inv);
            if (ct2 == CT - 1) write_head(h);
        }
    }
}

}  // namespace

hipError_t launch_path_transition(TransArgs a, hipStream_t s) {
    a.ntile = (a.L + kTok - 1) / kTok;
    const dim3 grid((unsigned)(a.B * a.ntile)), block(256);
    if (a.D == 64 && a.R == 64) hipLaunchKernelGGL((path_transition_kernel<64, 64>), grid, block, 0, s, a);
    else if (a.D == 64 && a.R == 32) hipLaunchKernelGGL((path_transition_kernel<64, 32>), grid, block, 0, s, a);
    else if (a.D == 128 && a.R == 64) hipLaunchKernelGGL((path_transition_kernel<128, 64>), grid, block, 0, s, a);
    else if (a.D == 128 && a.R == 32) hipLaunchKernelGGL((path_transition_kernel<128, 32>), grid, block, 0, s, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace path

using namespace path;

extern "C" int path_transition_prep(const void* x, const void* w_down, const void* w_up,
                                    const float* conv, const void* u, const float* b, void* w,
                                    float* beta, int B, int L, int Dm, int r, int H, int d,
                                    int dtype, void* stream) {
    if (B < 1 || L < 1 || Dm < 1 || r < 1 || H < 1 || d < 1) return PATH_ERR_INVALID;
    if (dtype != PATH_F32 && dtype != PATH_BF16) return PATH_ERR_INVALID;
    if (!x || !w_down || !w_up || !conv || !u || !b || !w || !beta) return PATH_ERR_INVALID;
    if (dtype != PATH_BF16) return PATH_ERR_UNSUPPORTED;
    if ((d != 64 && d != 128) || (r != 32 && r != 64) || r + H > 128 || Dm % kKc != 0)
        return PATH_ERR_UNSUPPORTED;
    if ((long long)B * H * L * d >= (1LL << 31) || (long long)B * L * Dm >= (1LL << 31))
        return PATH_ERR_UNSUPPORTED;
    TransArgs a{};
    a.x = x; a.w_down = w_down; a.w_up = w_up; a.conv = conv; a.u = u; a.b = b;
    a.w = w; a.beta = beta;
    a.B = B; a.L = L; a.Dm = Dm; a.R = r; a.H = H; a.D = d;
    return launch_path_transition(a, static_cast<hipStream_t>(stream)) == hipSuccess
               ? PATH_OK : PATH_ERR_HIP;
}
