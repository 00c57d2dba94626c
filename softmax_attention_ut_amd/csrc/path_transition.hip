// Transition parameters of every token from the layer input (Chinese notes,
// "key design"; Dutch summary section 2, "Kernmechanisme"):
//     z_t = W_up (W_down x_t),  c_t = conv0 * z_t + conv1 * z_{t-1} + conv2 * z_{t-2},
//     w_t = per-head L2 normalisation of c_t,  beta_t = 2 sigmoid(u . x_t + b).
//
// One 256-thread workgroup per tile of 64 consecutive tokens of one sequence.
// The first two rows of a tile are the convolution's reach into the tile
// before (recomputed, not written), so tiles start 62 tokens apart and every
// token's w depends only on its own workgroup.
//
// Stage 1 (HBM-bound: every element of x is read once):
//     [W_down; u] (r + H channels) x x^T on 16x16x32 bf16 MFMA, fp32
//     accumulators.  x is staged in LDS 128 columns at a time (double
//     buffered, one barrier per stage) and read as the B operand by all four
//     waves; wave q computes channel tiles q and q + 4 for all 64 tokens, with
//     its weight rows read from global memory (they are shared by every
//     workgroup and stay in L2).  Channels < r are y = W_down x; the rest give
//     beta.  y goes to LDS as a bf16 (high, low) pair.
// Stage 2 (per head, one wave per head):
//     W_up[head] x y^T on MFMA (high and low parts of y), so a lane holds one
//     token and four consecutive channels.  The convolution along tokens is a
//     shift across the 16 lanes of a DPP row (the previous token tile supplies
//     the first lanes), the squared norm is summed over the lane's channels
//     and across the four lane groups, and the normalised bf16 rows are
//     staged in LDS and written as whole 16-byte units.
#include "path_attn.h"
#include "path_internal.h"

namespace path {

namespace {

constexpr int kTok = 64;               // token rows per workgroup
constexpr int kHalo = 2;               // the convolution reaches two tokens back
constexpr int kOut = kTok - kHalo;     // tokens written per workgroup
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
constexpr int kRowShr = 0x110;   // + n: lane j reads lane j - n (j < n: invalid)
constexpr int kRowRor = 0x120;   // + n: lane j reads lane (j - n) mod 16

template <int N>
__device__ __forceinline__ float row_ror(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v),
                                                              kRowRor + N, 0xf, 0xf, true));
}

// lane j >= N of a row gets cur from lane j - N; lanes j < N keep `old`
template <int N>
__device__ __forceinline__ float row_shr(float cur, float old) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        __builtin_bit_cast(int, old), __builtin_bit_cast(int, cur), kRowShr + N, 0xf, 0xf,
        false));
}

template <int D, int R>
__global__ __launch_bounds__(256, 2) void path_transition_kernel(const TransArgs a) {
    constexpr int XROW = kKc * 2;                  // bytes per staged x row
    constexpr int XBUF = kTok * XROW;              // one x stage
    constexpr int YROW = 2 * R + 16;               // bytes per y row (padded)
    constexpr int SROW = 2 * D + 16;               // bytes per output staging row
    constexpr int SBUF = kTok * SROW;              // one wave's output staging
    constexpr int REGION = (2 * XBUF > 4 * SBUF) ? 2 * XBUF : 4 * SBUF;
    constexpr int KS = R / 32;                     // k-steps of the second product
    constexpr int CT = D / 16;                     // channel tiles of a head
    __shared__ __align__(16) char lds[REGION + 2 * kTok * YROW];
    char* const xs = lds;                          // x stages, later the output staging
    char* const yhi = lds + REGION;
    char* const ylo = yhi + kTok * YROW;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int seq = blockIdx.x / a.ntile, tile = blockIdx.x % a.ntile;
    const int t0 = tile * kOut - kHalo;            // token of local row 0
    const int L = a.L, Dm = a.Dm, H = a.H;
    const bf16* const x = static_cast<const bf16*>(a.x) + (size_t)seq * L * Dm;

    // ---- stage 1: [W_down; u] x^T ---------------------------------------
    // x copy: 64 rows x 16 units of 16 bytes per stage, 4 units per thread;
    // unit un of row rr is stored at unit un ^ (rr & 15) (conflict-free reads)
    bf16x8 pre[4];
    auto load_x = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = tid + 256 * i, rr = p >> 4, un = p & 15, t = t0 + rr;
            pre[i] = (t >= 0 && t < L) ? ld8(x + (size_t)t * Dm + k0 + 8 * un) : zero8();
        }
    };
    auto store_x = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = tid + 256 * i, rr = p >> 4, un = p & 15;
            *reinterpret_cast<bf16x8*>(xs + buf * XBUF + rr * XROW + ((un ^ (rr & 15)) << 4)) =
                pre[i];
        }
    };

    // this wave's channel tiles q and q + 4: lane row = channel 16 * tile + col
    const int nch = R + H;
    const bf16* src[2];
    bool live[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int ct = wave + 4 * c, ch = 16 * ct + col;
        live[c] = 16 * ct < nch;                   // wave-uniform
        src[c] = ch < R ? static_cast<const bf16*>(a.w_down) + (size_t)ch * Dm
               : ch < nch ? static_cast<const bf16*>(a.u) + (size_t)(ch - R) * Dm
               : nullptr;
    }
    auto load_w = [&](bf16x8 (&wa)[2][4], int k0) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                wa[c][ks] = (live[c] && src[c]) ? ld8(src[c] + k0 + 32 * ks + 8 * grp) : zero8();
    };

    f32x4 acc[2][4];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[c][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = Dm / kKc;
    bf16x8 wcur[2][4], wnext[2][4];
    load_x(0);
    load_w(wcur, 0);
    store_x(0);
    __syncthreads();
    for (int kc = 0; kc < nk; ++kc) {
        const int buf = kc & 1;
        const bool more = kc + 1 < nk;
        if (more) {
            load_x((kc + 1) * kKc);
            load_w(wnext, (kc + 1) * kKc);
        }
        const char* xb = xs + buf * XBUF;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x8 xv[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const int rr = 16 * tt + col;
                xv[tt] = *reinterpret_cast<const bf16x8*>(xb + rr * XROW +
                                                          (((4 * ks + grp) ^ (rr & 15)) << 4));
            }
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                if (!live[c]) continue;
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) acc[c][tt] = mfma16(wcur[c][ks], xv[tt], acc[c][tt]);
            }
        }
        if (more) {
            store_x(buf ^ 1);
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) wcur[c][ks] = wnext[c][ks];
        }
        __syncthreads();
    }

    // accumulator (c, tt) register i: channel 16 * (wave + 4c) + 4 grp + i, local token 16 tt + col
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int ct = wave + 4 * c;
        if (!live[c]) continue;
        if (16 * ct < R) {
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                bf16x4 hi, lo;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float v = acc[c][tt][i];
                    hi[i] = static_cast<bf16>(v);
                    lo[i] = static_cast<bf16>(v - static_cast<float>(hi[i]));
                }
                const int off = (16 * tt + col) * YROW + (16 * ct + 4 * grp) * 2;
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
                    const int rr = 16 * tt + col, t = t0 + rr;
                    if (rr >= kHalo && t < L)
                        bout[t] = 2.f / (1.f + expf(-(acc[c][tt][i] + bh)));
                }
            }
        }
    }
    __syncthreads();

    // ---- stage 2: per head, W_up[head] y^T, convolution, norm ------------
    bf16x8 yb[4][KS][2];                           // the same B operands for every head
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int off = (16 * tt + col) * YROW + (32 * ks + 8 * grp) * 2;
            yb[tt][ks][0] = *reinterpret_cast<const bf16x8*>(yhi + off);
            yb[tt][ks][1] = *reinterpret_cast<const bf16x8*>(ylo + off);
        }

    char* const stg = xs + wave * SBUF;
    const bf16* const wup = static_cast<const bf16*>(a.w_up);
    const int nrows = min(kTok, L - t0) - kHalo;   // tokens of this tile that exist

    // convolved channels 16 ct2 + 4 grp + i of local tokens 16 tt + col
    auto conv_tile = [&](int h, int ct2, f32x4 (&cv)[4]) {
        const int e = h * D + 16 * ct2;
        bf16x8 wu[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) wu[ks] = ld8(wup + (size_t)(e + col) * R + 32 * ks + 8 * grp);
        float tap[4][3];
        const float* const cp = a.conv + (size_t)(e + 4 * grp) * 3;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int k = 0; k < 3; ++k) tap[i][k] = cp[3 * i + k];
        f32x4 z[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            z[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                z[tt] = mfma16(wu[ks], yb[tt][ks][0], z[tt]);
                z[tt] = mfma16(wu[ks], yb[tt][ks][1], z[tt]);
            }
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float cur = z[tt][i];
                // tokens one and two back: this row shifted, the first lanes
                // from the previous token tile (row 0 has none: those lanes are
                // the halo, whose outputs are not written)
                const float p1 = tt ? row_ror<1>(z[tt ? tt - 1 : 0][i]) : 0.f;
                const float p2 = tt ? row_ror<2>(z[tt ? tt - 1 : 0][i]) : 0.f;
                const float s1 = row_shr<1>(cur, p1);
                const float s2 = row_shr<2>(cur, p2);
                cv[tt][i] = tap[i][0] * cur + tap[i][1] * s1 + tap[i][2] * s2;
            }
    };

    for (int h = wave; h < H; h += 4) {
        // the channel tiles are computed twice, first for the squared norm,
        // then for the values (keeping them all live would double the
        // register file this needs and halve the workgroups per CU)
        float ss[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int ct2 = 0; ct2 < CT; ++ct2) {
            f32x4 cv[4];
            conv_tile(h, ct2, cv);
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) ss[tt] += cv[tt][i] * cv[tt][i];
        }
        float inv[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            float s = ss[tt];
            s += __shfl_xor(s, 16);
            s += __shfl_xor(s, 32);
            inv[tt] = s > 0.f ? 1.f / sqrtf(s) : 0.f;
        }
#pragma unroll 1
        for (int ct2 = 0; ct2 < CT; ++ct2) {
            f32x4 cv[4];
            conv_tile(h, ct2, cv);
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                bf16x4 o;
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = static_cast<bf16>(cv[tt][i] * inv[tt]);
                *reinterpret_cast<bf16x4*>(stg + (16 * tt + col) * SROW + (16 * ct2 + 4 * grp) * 2) = o;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // rows kHalo .. kHalo + nrows - 1 form one contiguous run of w[seq][h]
        bf16* const wout = static_cast<bf16*>(a.w) + (((size_t)seq * H + h) * L + t0 + kHalo) * D;
        const int units = nrows * (D / 8);
        for (int q = lane; q < units; q += 64) {
            const int rr = q / (D / 8), un = q % (D / 8);
            *reinterpret_cast<bf16x8*>(wout + (size_t)q * 8) =
                *reinterpret_cast<const bf16x8*>(stg + (rr + kHalo) * SROW + un * 16);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

}  // namespace

hipError_t launch_path_transition(TransArgs a, hipStream_t s) {
    a.ntile = (a.L + kOut - 1) / kOut;
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
