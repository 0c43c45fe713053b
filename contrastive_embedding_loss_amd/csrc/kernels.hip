// Device kernels of the fused Matryoshka contrastive loss for gfx950 (MI355X).
//
// Pages (cited by title and section):
//  * "Scaling-Up Contrastive Learning over NVLink Multicast", "One Set or Two":
//    CLIP row softmax, the SigLIP equation, five Matryoshka grids.
//  * Same page, "On the Chip: Tensor Memory & the Matryoshka Sweep": one sweep
//    over the embedding serves all prefixes; per-cell normalisation with stored
//    inverse norms; band gradients built as running sums; the grid never leaves
//    the chip; per-tile partials folded afterwards.
//  * UForm README, training-stack paragraphs: BF16 operands, FP32 accumulation,
//    FP32 log-sum-exps and partial-gradient slabs.
//
// Notation used throughout: outer rows X (the rows whose gradient a pass owns)
// against inner rows Y.  The row pass has X = q, Y = k; the column pass has
// X = k, Y = q.  S^p = <x[:P_p], y[:P_p]>, logits in base-2 units
// u = l * log2(e); softmax kinds use one fixed shift c = -|s| log2(e) so that
// x = (l - b - |s|) log2(e) <= 0 and one exp per cell serves row and column sums.
#include <climits>
#include <type_traits>

#include "common.h"

namespace uform {

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// ----------------------------------------------------------------------------
// small helpers
// ----------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(unsigned int v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(unsigned int v) { return __uint_as_float(v & 0xffff0000u); }

__device__ __forceinline__ f16x8 pack_f16x8(const float (&v)[8]) {
    f16x8 r;
#pragma unroll
    for (int t = 0; t < 8; ++t) r[t] = (_Float16)v[t];
    return r;
}

// Sum over the 32 lanes of each wave half of v[lane & 31]: a reduce-scatter
// butterfly (31 exchanges instead of 32 x 5) without LDS traffic.  Stage 16
// uses v_permlane16_swap (rows of 16 lanes trade halves); stages 8 and 4 pair
// lane i with 15 - i and 7 - i (DPP row mirror and half mirror), stages 2 and
// 1 use quad permutes.  Each stage pairs lanes that differ in the stage's bit
// and agree on the bits of the stages before, so lane l keeps slot l & 31.
// A lane permutation within rows of 16 (every source lane exists, so the zero that bound_ctrl
// gives a missing source never appears); in this form the compiler folds it into the add that
// consumes it (v_add_f32 with a DPP operand instead of a move and an add).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float reduce_scatter32(float (&v)[32], int lane) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[i]), __float_as_uint(v[i + 16]), false, false);
        v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    auto stage = [&](auto hc, auto cc) {
        constexpr int h = decltype(hc)::value, C = decltype(cc)::value;
        const bool up = (lane & h) != 0;
#pragma unroll
        for (int i = 0; i < h; ++i) {
            const float keep = up ? v[i + h] : v[i];
            const float send = up ? v[i] : v[i + h];
            v[i] = keep + dpp<C>(send);
        }
    };
    stage(std::integral_constant<int, 8>{}, std::integral_constant<int, 0x140>{});  // row_mirror
    stage(std::integral_constant<int, 4>{}, std::integral_constant<int, 0x141>{});  // row_half_mirror
    stage(std::integral_constant<int, 2>{}, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
    stage(std::integral_constant<int, 1>{}, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
    return v[0];
}
// Sum over the wave, in every lane, without LDS round trips: quad permutes (lanes 1 and 2 apart),
// the half-row and row mirrors, then the 16-lane and 32-lane swaps add the partner row and the
// partner half-wave.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp<0xB1>(v);   // quad_perm [1, 0, 3, 2]
    v += dpp<0x4E>(v);   // quad_perm [2, 3, 0, 1]
    v += dpp<0x141>(v);  // row_half_mirror
    v += dpp<0x140>(v);  // row_mirror
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(h[0]) + __uint_as_float(h[1]);
}

__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
template <int N>
__device__ __forceinline__ void wait_vm_n() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// barrier that waits for this wave's LDS accesses only (not for its outstanding global loads)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Direct global -> LDS copies issued from inline assembly: the compiler does not
// see them, so it adds no waits of its own before LDS accesses; the caller waits
// for them with s_waitcnt vmcnt.  The LDS destination (M0) must be wave-uniform.
// dma_row1 / dma_row2: one inner row of 1 KB or 2 KB, 16 bytes per lane from
// base + voff into LDS at m0v + 16 lane (the instruction offset moves the source
// and the LDS destination alike).  dma4_m0: 4 bytes per lane from g into m0v + 4 lane.
__device__ __forceinline__ void dma_row1(const void *base, uint32_t voff, uint32_t m0v) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(m0v) : "memory");
}
__device__ __forceinline__ void dma_row2(const void *base, uint32_t voff, uint32_t m0v) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1\n\tglobal_load_lds_dwordx4 %0, %1 offset:1024" ::"v"(
                     voff),
                 "s"(base), "s"(m0v)
                 : "memory");
}
// the same with M0 = ma + mb (two scalar operands, one scalar add)
__device__ __forceinline__ void dma_row1_add(const void *base, uint32_t voff, uint32_t ma, uint32_t mb) {
    asm volatile("s_add_u32 m0, %2, %3\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(ma), "s"(mb)
                 : "memory");
}
__device__ __forceinline__ void dma_row2_add(const void *base, uint32_t voff, uint32_t ma, uint32_t mb) {
    asm volatile("s_add_u32 m0, %2, %3\n\tglobal_load_lds_dwordx4 %0, %1\n\tglobal_load_lds_dwordx4 %0, %1 offset:1024" ::"v"(
                     voff),
                 "s"(base), "s"(ma), "s"(mb)
                 : "memory");
}
__device__ __forceinline__ void dma4_add(const void *g, uint32_t ma, uint32_t mb) {
    asm volatile("s_add_u32 m0, %1, %2\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(ma), "s"(mb) : "memory");
}
__device__ __forceinline__ void dma4_m0(const void *g, uint32_t m0v) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(m0v) : "memory");
}

// ----------------------------------------------------------------------------
// k_prep: per-prefix inverse L2 norms of every row (and s log2(e) times
// them), the exact power-of-two row scale sig ~ 1/|row| and the backward's
// per-row operand scale gam; for query rows of the sigmoid kinds also the prefix dot products
// with their positive key (the softmax kinds' forward takes them from its diagonal tiles, so
// that each row is read once here).  A workgroup takes 4 RPW consecutive rows of the
// list (query rows, then key rows), a wave RPW of them (16, 4 or 1: enough
// workgroups to fill the GPU), one at a time with the next row's loads in flight.  Lane l holds the 16-byte chunks
// l, l + 64, ... of a row (NC of them: D <= 512 NC); prefix ends are multiples of 32, so no
// chunk straddles one, and the sum over a prefix is an inclusive scan over the chunks read at
// the prefix's last chunk.  Results go through LDS so that the tables are
// written with consecutive rows on consecutive lanes.
// ----------------------------------------------------------------------------
constexpr int kPrepRows = 64;  // most rows per workgroup

// inclusive prefix sum over the 64 lanes, in DPP moves (no LDS round trips): shifts by 1, 2, 4, 8
// inside each row of 16 lanes (lanes shifted in from outside the row read 0), then lane 15 of
// each row added to the row after it and lane 31 to rows 2 and 3
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_in(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xf, true));
}
__device__ __forceinline__ float wave_scan(float v, int) {
    v += dpp_in<0x111, 0xf>(v);  // row_shr:1
    v += dpp_in<0x112, 0xf>(v);  // row_shr:2
    v += dpp_in<0x114, 0xf>(v);  // row_shr:4
    v += dpp_in<0x118, 0xf>(v);  // row_shr:8
    v += dpp_in<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp_in<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

__device__ __forceinline__ float sq8(const uint4 &a) {
    const unsigned int w[4] = {a.x, a.y, a.z, a.w};
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) s = fmaf(bf16_lo(w[c]), bf16_lo(w[c]), fmaf(bf16_hi(w[c]), bf16_hi(w[c]), s));
    return s;
}
__device__ __forceinline__ float dot8(const uint4 &a, const uint4 &b) {
    const unsigned int u[4] = {a.x, a.y, a.z, a.w}, v[4] = {b.x, b.y, b.z, b.w};
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) s = fmaf(bf16_lo(u[c]), bf16_lo(v[c]), fmaf(bf16_hi(u[c]), bf16_hi(v[c]), s));
    return s;
}

template <int RPW, int NC>
__global__ __launch_bounds__(256) void k_prep(PrepArgs a) {
    constexpr int RB = 4 * RPW;  // rows per workgroup
    __shared__ float res[RB][2 * kMaxP + 1];  // per row: inv[P] | posdot[P] | sig
    if (blockIdx.x == 0 && threadIdx.x < 4 * a.pf.n) a.gmax[threadIdx.x] = 0.f;  // k_maxes' start
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t rows = a.R + a.N, g0 = (int64_t)blockIdx.x * RB;
    const int D = a.D, P = a.pf.n, nch = D / 8;
    // this lane's prefix (lane < P): its chunk count
    int m = 1;
#pragma unroll
    for (int p = 0; p < kMaxP; ++p)
        if (p < P && lane == p) m = a.pf.w[p] / 8;
    uint4 bx[2][NC], by[2][NC];
    auto fetch = [&](int j, int s) {
        const int64_t g = g0 + RPW * wave + j;
        const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int c = 0; c < NC; ++c) bx[s][c] = by[s][c] = z;
        if (g >= rows) return;
        const bool isq = g < a.R;
        const u16 *x = isq ? a.q + g * D : a.k + (g - a.R) * D;
#pragma unroll
        for (int c = 0; c < NC; ++c)
            if (lane + 64 * c < nch) bx[s][c] = *(const uint4 *)(x + 8 * (lane + 64 * c));
        if (isq && a.want_pos) {
            const u16 *y = a.k + ((g + a.off) ^ a.pxor) * D;
#pragma unroll
            for (int c = 0; c < NC; ++c)
                if (lane + 64 * c < nch) by[s][c] = *(const uint4 *)(y + 8 * (lane + 64 * c));
        }
    };
    fetch(0, 0);
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
        if (j + 1 < RPW) fetch(j + 1, (j + 1) & 1);
        const int64_t g = g0 + RPW * wave + j;
        if (g >= rows) continue;  // wave-uniform
        const int s = j & 1;
        // lane p < P: sums over prefix p's chunks, group by group of 64 chunks (a group's total at
        // lane 63).  Every lane takes part in every shuffle (a lane outside the exec mask supplies
        // no value).
        float ss = 0.f, dt = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const float Sc = wave_scan(sq8(bx[s][c]), lane);
            const float Tc = a.want_pos ? wave_scan(dot8(bx[s][c], by[s][c]), lane) : 0.f;
            const int at = min(max(m - 64 * c, 1), 64) - 1;
            const float av = __shfl(Sc, at), bv = __shfl(Tc, at);
            ss += m > 64 * c ? av : 0.f;
            dt += m > 64 * c ? bv : 0.f;
        }
        const int r = RPW * wave + j;
        if (lane < P) {
            res[r][lane] = 1.0f / sqrtf(fmaxf(ss, 1.17549435e-38f));
            res[r][kMaxP + lane] = dt;
        }
        // the row scale sig = 2^-floor(log2 |row[:P_n]|), formed by every lane from lane P - 1's sum
        const float ssP = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ss), P - 1));
        const float normP = sqrtf(ssP);
        const float sig = normP > 0.f ? ldexpf(1.0f, -ilogbf(normP)) : 1.0f;
        if (lane == 0) res[r][2 * kMaxP] = sig;
        if (a.qH) {
            // the backward's FP16 copy of the row, times sig (exact: a power of two, and a BF16 value
            // times it fits FP16 above FP16's subnormal range)
            const bool isq = g < a.R;
            _Float16 *xh = isq ? a.qH + g * D : a.kH + (g - a.R) * D;
#pragma unroll
            for (int c = 0; c < NC; ++c)
                if (lane + 64 * c < nch) {
                    const unsigned int in[4] = {bx[s][c].x, bx[s][c].y, bx[s][c].z, bx[s][c].w};
                    f16x8 h;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        h[2 * i] = (_Float16)(bf16_lo(in[i]) * sig);
                        h[2 * i + 1] = (_Float16)(bf16_hi(in[i]) * sig);
                    }
                    *(f16x8 *)(xh + 8 * (lane + 64 * c)) = h;
                }
        }
    }
    // zero rows past the last row of each copy (block 0: q's; k's by block 1, or by block 0 in a
    // grid of one block)
    if (a.qH)
        for (int which = 0; which < 2; ++which) {
            if ((int)blockIdx.x != (gridDim.x > 1 ? which : 0)) continue;
            _Float16 *xh = which == 0 ? a.qH : a.kH;
            const int64_t e0 = (which == 0 ? a.R : a.N) * D, e1 = (which == 0 ? a.Rpad : a.Npad) * D;
            for (int64_t e = e0 + 8 * (int64_t)threadIdx.x; e < e1; e += 8 * 256) *(f16x8 *)(xh + e) = f16x8{};
        }
    __syncthreads();
    // tables [p][row]: consecutive rows on consecutive lanes (two runs where the block holds both kinds)
    for (int e = threadIdx.x; e < RB * (P + 1); e += 256) {
        const int p = e / RB, r = e % RB;
        const int64_t g = g0 + r;
        if (g >= rows) continue;
        const bool isq = g < a.R;
        const int64_t i = isq ? g : g - a.R, nr = isq ? a.R : a.N;
        const float sig = res[r][2 * kMaxP];
        if (p < P) {
            const float inv = res[r][p];
            (isq ? a.invq : a.invk)[p * nr + i] = inv;
            (isq ? a.qA : a.kA)[p * nr + i] = a.a_scale * inv;
            (isq ? a.qIYR : a.kIYR)[p * nr + i] = inv / sig;
            if (isq && a.want_pos) a.posdot[p * a.R + i] = res[r][kMaxP + p];
        } else {
            (isq ? a.sigq : a.sigk)[i] = sig;
            (isq ? a.gamq : a.gamk)[i] = a.gam_scale * res[r][P - 1];
        }
    }
}

// ----------------------------------------------------------------------------
// k_fwd: softmax forward.  One 128 x 128 tile of (query i, key j) per
// workgroup, 4 waves of 64 x 64 (2 x 2 MFMA 32x32x16 blocks each), operands
// copied global -> LDS directly in 64-wide slices of d, one slice ahead (two
// workgroups per CU; one barrier per slice).  At every prefix boundary the
// FP32 accumulators are read in place ("snapshotted") and each cell's
// e = 2^(S a_i ik_j + c) is added to a row partial and a column partial; the
// positive cell is left out of both, and the masked tiles (which hold every
// positive cell) write its raw prefix dot product to posdot, from which the
// statistics kernels add it back in FP32.  Each wave keeps its reduced partials (one row
// and one column value per lane and prefix) until the sweep ends; then the two
// waves that share a row (a column) add theirs through LDS and the tile writes
// one partial per row and per column: rowpart[jt][p][i], colpart[it][p][j].
// ----------------------------------------------------------------------------
constexpr int FB = 128;
constexpr int FK = 64;

// A snapshot of prefix p: this lane's row sum (row fwd_lane_row(wi, lane) of the tile, over the
// wave's 64 columns) into rkeep[p] and its column sum (column 64 wj + lane, over the wave's 64
// rows) into ckeep[p].
__device__ __forceinline__ int fwd_lane_row(int wi, int lane) {
    const int v = lane & 31, bi = v >> 4, r = v & 15;
    return wi * 64 + bi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

template <bool MASKED>
__device__ __forceinline__ void fwd_snapshot(const f32x16 (&acc)[2][2], int p, int wi, int wj, int lane, int tid,
                                             int64_t i0, int64_t j0, int64_t R, int64_t N, int64_t off, int P,
                                             float cshift, const float (*fA)[FB], const float (*fI)[FB],
                                             float (&rkeep)[kMaxP], float (&ckeep)[kMaxP], float *posdot) {
    float rs[32];
    float cs[2];
    float Ij[2];
    int64_t gj[2];
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
        const int jl = wj * 64 + bj * 32 + (lane & 31);
        Ij[bj] = fI[p][jl];
        gj[bj] = j0 + jl;
    }
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int il = wi * 64 + bi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const float Ai = fA[p][il];
            float e[2];
#pragma unroll
            for (int bj = 0; bj < 2; ++bj) {
                e[bj] = __builtin_amdgcn_exp2f(fmaf(acc[bi][bj][r] * Ai, Ij[bj], cshift));
                if (MASKED) {
                    const int64_t gi = i0 + il;
                    const bool ok = (gi < R) & (gj[bj] < N) & (gj[bj] != gi + off);
                    e[bj] = ok ? e[bj] : 0.f;
                    // the positive cell (gi, off + gi) is in a masked tile: its prefix dot product, as the
                    // MFMAs summed it, is the positive's logit input for the statistics and the backward
                    if ((gi < R) & (gj[bj] == gi + off)) posdot[p * R + gi] = acc[bi][bj][r];
                }
                cs[bj] = (bi == 0 && r == 0) ? e[bj] : cs[bj] + e[bj];  // no addition of a zero start
            }
            rs[bi * 16 + r] = e[0] + e[1];
        }
    }
    // row sums: lane (lane & 31) of each half ends up with row index v = lane & 31
    const float rv = reduce_scatter32(rs, lane);
    // column sums of this wave's 64 rows: lanes 0..31 column block 0, 32..63 block 1
    const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(cs[0]), __float_as_uint(cs[1]), false, false);
    const float cv = __uint_as_float(c[0]) + __uint_as_float(c[1]);
#pragma unroll
    for (int q = 0; q < kMaxP; ++q)
        if (q == p) {
            rkeep[q] = rv;
            ckeep[q] = cv;
        }
}

// The tile's partials: the two waves of a row (of a column) add theirs in LDS (the operand ring,
// free after the sweep), and the tile writes one partial per row and per column.
__device__ __forceinline__ void fwd_write_partials(float *lds, const float (&rkeep)[kMaxP], const float (&ckeep)[kMaxP],
                                                   int wi, int wj, int lane, int tid, int P, int64_t i0, int64_t j0,
                                                   int64_t R, int64_t N, int64_t it, int64_t jt,
                                                   float *__restrict__ rowpart, float *__restrict__ colpart) {
    float *rl = lds, *cl = lds + 2 * kMaxP * FB;  // [2][kMaxP][FB] each
    lds_barrier();  // every wave is done with the ring
    const int il = fwd_lane_row(wi, lane);
#pragma unroll
    for (int p = 0; p < kMaxP; ++p)
        if (p < P) {
            rl[(wj * kMaxP + p) * FB + il] = rkeep[p];
            cl[(wi * kMaxP + p) * FB + wj * 64 + lane] = ckeep[p];
        }
    lds_barrier();
    for (int e = tid; e < P * FB; e += 256) {
        const int p = e / FB, x = e % FB;
        if (i0 + x < R) rowpart[(jt * P + p) * R + i0 + x] = rl[p * FB + x] + rl[(kMaxP + p) * FB + x];
        if (j0 + x < N) colpart[(it * P + p) * N + j0 + x] = cl[p * FB + x] + cl[(kMaxP + p) * FB + x];
    }
}

// Slices (64 wide) covered by the prefixes of ladder MASK (bit ds: a prefix ends at 32 (ds + 1)),
// for ladders whose prefixes all end on a slice boundary; 0 otherwise.
constexpr int fwd_ladder_slices(uint64_t mask) {
    if (mask == 0ull || (mask & 0x5555555555555555ull) != 0ull) return 0;
    return (64 - __builtin_clzll(mask)) / 2;
}
constexpr uint64_t fwd_ladder(uint64_t mask) { return fwd_ladder_slices(mask) > 0 ? mask : 0ull; }

template <uint64_t MASK>
__global__ __launch_bounds__(256, 2) void k_fwd(const u16 *__restrict__ q, const u16 *__restrict__ k, int64_t R,
                                                int64_t N, int D, Prefixes pf, int64_t off,
                                                const float *__restrict__ rowA, const float *__restrict__ colI,
                                                float cshift, float *__restrict__ rowpart,
                                                float *__restrict__ colpart, float *__restrict__ posdot) {
    // Operand slices (128 rows x 64 bf16, 128 bytes per row) in a ring of two, copied
    // global -> LDS directly one slice ahead.  Rows are unpadded; the 16-byte chunk c of
    // row r sits at position c ^ ((r >> 1) & 7), so the MFMA operand reads (16 rows,
    // one chunk each per 16 lanes) meet 64 different banks.
    constexpr int SLB = FB * FK * 2;  // bytes per operand slice
    __shared__ __attribute__((aligned(16))) u16 Ring[2][2][FB * FK];  // [slot][q | k]
    __shared__ float fA[kMaxP][FB];
    __shared__ float fI[kMaxP][FB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wi = wave >> 1, wj = wave & 1;
    int64_t it, jt;
    {
        // Workgroups are dealt to the 8 XCDs in turn (id mod 8).  Give each XCD a contiguous
        // run of tiles in grouped order (8 row tiles, then the next column), so that the tiles
        // resident on one XCD share 8 row tiles and 8 column tiles in its L2.
        const int64_t nIt = (R + FB - 1) / FB, nJt = (N + FB - 1) / FB, T = nIt * nJt;
        const int64_t L = blockIdx.x, x = L % 8, idx = L / 8;
        const int64_t base = (T / 8) * x + (x < T % 8 ? x : T % 8);  // tiles of the XCDs before x
        const int64_t t = base + idx;
        constexpr int64_t GM = 8;
        const int64_t per_group = GM * nJt, g = t / per_group, i0g = g * GM;
        const int64_t gsz = nIt - i0g < GM ? nIt - i0g : GM;
        it = i0g + (t % per_group) % gsz;
        jt = (t % per_group) / gsz;
    }
    const int64_t i0 = it * FB, j0 = jt * FB;
    const int P = pf.n;
    const int Dsw = pf.w[P - 1];

    for (int e = tid; e < P * FB; e += 256) {
        const int p = e / FB, r = e % FB;
        fA[p][r] = (i0 + r < R) ? rowA[p * R + i0 + r] : 0.f;
        fI[p][r] = (j0 + r < N) ? colI[p * N + j0 + r] : 0.f;
    }
    const bool masked = (i0 + FB > R) || (j0 + FB > N) || ((j0 < i0 + off + FB) && (i0 + off < j0 + FB));

    // copies: this wave moves pieces 4 wave .. 4 wave + 3 (8 rows x 128 bytes each) of both
    // operands; lane l of piece pc fills row 8 pc + (l >> 3), position l & 7 (rows past the
    // end repeat the last row: finite values in cells that are masked)
    uint32_t vq[4], vk[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int row = 8 * (4 * wave + c) + (lane >> 3);
        const uint32_t ch = (uint32_t)((lane & 7) ^ ((row >> 1) & 7));
        const int64_t rq = i0 + row < R ? row : R - 1 - i0, rk = j0 + row < N ? row : N - 1 - j0;
        vq[c] = (uint32_t)rq * (uint32_t)D * 2u + 16u * ch;
        vk[c] = (uint32_t)rk * (uint32_t)D * 2u + 16u * ch;
    }
    const uint32_t ring_lds = (uint32_t)(uintptr_t)&Ring[0][0][0];
    const u16 *qt = q + i0 * D, *kt = k + j0 * D;  // tile row bases (wave-uniform)
    auto issue = [&](int st) {
        const int slot = st & 1;
        const u16 *qs = qt + st * FK, *ks_ = kt + st * FK;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t m = ring_lds + (uint32_t)(slot * 2 * SLB + 1024 * (4 * wave + c));
            dma_row1(qs, vq[c], m);
            dma_row1(ks_, vk[c], m + SLB);
        }
    };

    // operand reads: rows wi 64 + b 32 + (lane & 31) (and wj for k); chunk 2 ks + (lane >> 5)
    const int rl = lane & 31, sw = (rl >> 1) & 7;
    const uint32_t rdq = (uint32_t)((wi * 64 + rl) * 128 + 16 * ((lane >> 5) ^ (sw & 1)));
    const uint32_t rdk = (uint32_t)((wj * 64 + rl) * 128 + 16 * ((lane >> 5) ^ (sw & 1))) + SLB;

    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
    float rkeep[kMaxP], ckeep[kMaxP];  // this lane's row and column partial of every prefix
#pragma unroll
    for (int q = 0; q < kMaxP; ++q) rkeep[q] = ckeep[q] = 0.f;

    if constexpr (MASK != 0ull) {
        // Prefix ladder known at compile time: no branch inside a slice.  The ring holds four
        // 32-wide slices (rows of 64 bytes; the 16-byte chunk c of row r at position
        // c ^ ((r >> 2) & 3), so the operand reads of 16 rows meet 64 different banks).  Per slice
        // st (slot st & 3): the operands of step 1 are read before the MFMAs of step 0; then one
        // barrier publishes slice st + 1 and frees slot st & 3 for the copies of slice st + 4
        // (three slices ahead), and the first operands of slice st + 1 are read before the MFMAs
        // of step 1.  Snapshots follow the slices where a prefix ends.
        constexpr int FK2 = 32;
        constexpr int SLB2 = FB * FK2 * 2;  // bytes per operand slice
        constexpr int NSL = 2 * fwd_ladder_slices(MASK);
        static_assert(NSL >= 2, "every prefix must end on a 64-wide boundary");
        constexpr int NPm = __builtin_popcountll(MASK);
        // copies: this wave moves pieces 2 wave, 2 wave + 1 (16 rows x 64 bytes each) of both operands
        uint32_t cq[2], ck[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int row = 16 * (2 * wave + c) + (lane >> 2);
            const uint32_t ch = (uint32_t)((lane & 3) ^ ((row >> 2) & 3));
            const int64_t rq = i0 + row < R ? row : R - 1 - i0, rk = j0 + row < N ? row : N - 1 - j0;
            cq[c] = (uint32_t)rq * (uint32_t)D * 2u + 16u * ch;
            ck[c] = (uint32_t)rk * (uint32_t)D * 2u + 16u * ch;
        }
        auto issue2 = [&](int st) {
            const uint32_t m = ring_lds + (uint32_t)((st & 3) * 2 * SLB2 + 2048 * wave);
            const u16 *qs = qt + st * FK2, *ks_ = kt + st * FK2;
            dma_row1(qs, cq[0], m);
            dma_row1(qs, cq[1], m + 1024);
            dma_row1(ks_, ck[0], m + SLB2);
            dma_row1(ks_, ck[1], m + SLB2 + 1024);
        };
        const int sw4 = (rl >> 2) & 3, h = lane >> 5;
        const uint32_t rq0 = (uint32_t)((wi * 64 + rl) * 64), rk0 = (uint32_t)((wj * 64 + rl) * 64) + SLB2;
        const uint32_t po0 = 16u * (uint32_t)(h ^ sw4), po1 = 16u * (uint32_t)((2 + h) ^ sw4);
        const char *ring0 = (const char *)&Ring[0][0][0];
        auto lread = [&](int st, auto ksc, bf16x8(&av)[2], bf16x8(&bv)[2]) {
            const char *sb = ring0 + (st & 3) * 2 * SLB2;
            const uint32_t o = decltype(ksc)::value == 0 ? po0 : po1;
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                av[b] = *(const bf16x8 *)(sb + rq0 + o + b * 32 * 64);
                bv[b] = *(const bf16x8 *)(sb + rk0 + o + b * 32 * 64);
            }
        };
        auto mfma4 = [&](const bf16x8(&av)[2], const bf16x8(&bv)[2]) {
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[a], bv[b], acc[a][b], 0, 0, 0);
        };
        constexpr std::integral_constant<int, 0> K0{};
        constexpr std::integral_constant<int, 1> K1{};
        issue2(0);
        issue2(1);
        issue2(2);
        if (NSL > 3) issue2(3);
        if (NSL > 3)
            wait_vm_n<12>();  // slice 0 landed (slices 1..3 may still be in flight)
        else
            wait_vm_n<8>();
        lds_barrier();
        bf16x8 av0[2], bv0[2], av1[2], bv1[2];
        lread(0, K0, av0, bv0);
        int st = 0;
        auto slice = [&](auto lastc) {
            constexpr bool LAST = decltype(lastc)::value;  // the ladder's final slice
            lread(st, K1, av1, bv1);
            __builtin_amdgcn_sched_barrier(0);
            mfma4(av0, bv0);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (!LAST) {
                // this wave's copies of slice st + 1 landed (those of st + 2 and st + 3 may be in flight)
                if (st + 3 < NSL)
                    wait_vm_n<8>();
                else if (st + 2 < NSL)
                    wait_vm_n<4>();
                else
                    wait_vm();
                lds_barrier();  // every wave's copies visible; every wave's reads of slot st & 3 done
                if (st + 4 < NSL) issue2(st + 4);
                lread(st + 1, K0, av0, bv0);
            }
            __builtin_amdgcn_sched_barrier(0);
            mfma4(av1, bv1);
            __builtin_amdgcn_sched_barrier(0);
            ++st;
        };
        static_for<0, NPm>([&](auto pc) {
            constexpr int p = decltype(pc)::value;
            // 32-wide slices up to the end of prefix p
            constexpr int endsl = [] {
                int c = -1;
                for (int ds = 0; ds < 64; ++ds)
                    if (MASK & (1ull << ds))
                        if (++c == p) return ds + 1;
                return 0;
            }();
            if constexpr (p + 1 < NPm) {
                for (; st < endsl;) slice(std::false_type{});
            } else {
                for (; st < endsl - 1;) slice(std::false_type{});
                slice(std::true_type{});
            }
            if (masked)
                fwd_snapshot<true>(acc, p, wi, wj, lane, tid, i0, j0, R, N, off, P, cshift, fA, fI, rkeep, ckeep, posdot);
            else
                fwd_snapshot<false>(acc, p, wi, wj, lane, tid, i0, j0, R, N, off, P, cshift, fA, fI, rkeep, ckeep, posdot);
        });
    } else {
    const int nst = (Dsw + FK - 1) / FK;
    int pnext = 0;
    issue(0);
    for (int st = 0; st < nst; ++st) {
        wait_vm();      // this wave's copies of slice st landed
        lds_barrier();  // every wave's copies visible; every wave done with slice st - 1's slot
        if (st + 1 < nst) issue(st + 1);
        const char *sb = (const char *)&Ring[st & 1][0][0];
        bf16x8 avn[2], bvn[2];
        auto lread = [&](int ks, bf16x8(&av)[2], bf16x8(&bv)[2]) {
            const uint32_t o = 16u * (uint32_t)((2 * ks) ^ (sw & 6));
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                av[b] = *(const bf16x8 *)(sb + rdq + o + b * 32 * 128);
                bv[b] = *(const bf16x8 *)(sb + rdk + o + b * 32 * 128);
            }
        };
        // operands of the next 16-wide step are read before the MFMAs of this one
        lread(0, avn, bvn);
#pragma unroll
        for (int ks = 0; ks < FK / 16; ++ks) {
            const int dk = st * FK + ks * 16;
            bf16x8 av[2] = {avn[0], avn[1]}, bv[2] = {bvn[0], bvn[1]};
            if (ks + 1 < FK / 16) lread(ks + 1, avn, bvn);
            if (dk < Dsw) {
#pragma unroll
                for (int a = 0; a < 2; ++a)
#pragma unroll
                    for (int b = 0; b < 2; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[a], bv[b], acc[a][b], 0, 0, 0);
                if (pnext < P && dk + 16 == pf.w[pnext]) {
                    if (masked)
                        fwd_snapshot<true>(acc, pnext, wi, wj, lane, tid, i0, j0, R, N, off, P, cshift, fA, fI, rkeep,
                                           ckeep, posdot);
                    else
                        fwd_snapshot<false>(acc, pnext, wi, wj, lane, tid, i0, j0, R, N, off, P, cshift, fA, fI, rkeep,
                                            ckeep, posdot);
                    ++pnext;
                }
            }
        }
    }
    }
    fwd_write_partials(reinterpret_cast<float *>(&Ring[0][0][0]), rkeep, ckeep, wi, wj, lane, tid, P, i0, j0, R, N,
                       it, jt, rowpart, colpart);
}

// ----------------------------------------------------------------------------
// Statistics for the softmax kinds (one thread per row / per column).
// Row i: Z_i = sum_j 2^{x_ij} (negatives from the forward partials plus the
// positive), CE_i = ln(1 + neg/e_pos), row LSE; and the per-prefix
// coefficient tables the backward reads.  Column j likewise.
// ----------------------------------------------------------------------------
__device__ __forceinline__ float ce_from(float neg, float epos, float x_pos, float Z) {
    const float r = neg / epos;
    return (r < 1e30f) ? log1pf(r) : (logf(Z) - x_pos * kLn2);
}

__device__ __forceinline__ void block_sum_write(float v, float *red /*[4]*/, float *dst) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    v = wave_sum(v);
    if (lane == 0) red[wave] = v;
    __syncthreads();
    if (threadIdx.x == 0) *dst = ((red[0] + red[1]) + red[2]) + red[3];
    __syncthreads();
}

// Sum of the per-tile partials of row (or column) r, prefix p: the W waves of a block (4, 8 or
// 16, by the number of partials) each take every W-th tile (kStatRows consecutive rows per
// wave, so the loads coalesce), then the waves' sums are added in a fixed order.
constexpr int kStatWaves = 16;  // most waves per block
inline int stat_waves(int64_t ntiles) { return ntiles >= 128 ? 16 : ntiles >= 64 ? 8 : 4; }
__device__ __forceinline__ float fold_partials(const float *part, int64_t ntiles, int P, int p, int64_t len,
                                               int64_t r, bool ok, float (*fold)[kStatRows]) {
    const int g = threadIdx.x / kStatRows, rl = threadIdx.x % kStatRows;
    float v = 0.f;
    if (ok) {
        // eight independent running sums (eight loads in flight per lane), added in a fixed order
        const int W = (int)(blockDim.x / 64);
        float u[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        int64_t t = g;
        for (; t + 7 * W < ntiles; t += 8 * W) {
            float x[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) x[k] = part[((t + W * k) * P + p) * len + r];
#pragma unroll
            for (int k = 0; k < 8; ++k) u[k] += x[k];
        }
        for (; t < ntiles; t += W) u[0] += part[(t * P + p) * len + r];
        v = ((u[0] + u[1]) + (u[2] + u[3])) + ((u[4] + u[5]) + (u[6] + u[7]));
    }
    fold[g][rl] = v;
    __syncthreads();
    float s = 0.f;
    for (int h = 0; h < (int)(blockDim.x / 64); h += 4)
        s += (fold[h][rl] + fold[h + 1][rl]) + (fold[h + 2][rl] + fold[h + 3][rl]);
    __syncthreads();
    return s;
}

// The loss partial of a statistics block: only wave 0 (the block's rows) holds terms.
__device__ __forceinline__ void lead_sum_write(float v, float *dst) {
    if (threadIdx.x < 64) {
        v = wave_sum(v);
        if (threadIdx.x == 0) *dst = v;
    }
}

// The lead threads (one per row) read every prefix's table entries of their row into LDS before
// the folds, so that those reads are in flight during the folds rather than after each of them
// (each lead thread reads back only what it wrote: no barrier).
__global__ __launch_bounds__(64 * kStatWaves, 8) void k_rowstats(StatsArgs a) {  // two blocks per CU
    __shared__ float fold[kStatWaves][kStatRows];
    __shared__ float tab[5][kMaxP][kStatRows];  // inv_q, inv_k of the positive, posdot, qA, qIYR
    const int rl = threadIdx.x % kStatRows;
    const int64_t i = (int64_t)blockIdx.x * kStatRows + rl;
    const bool lead = threadIdx.x < kStatRows;
    const bool mine = lead && i < a.R;
    const int P = a.pf.n;
    if (mine)
        for (int p = 0; p < P; ++p) {
            tab[0][p][rl] = a.invq[p * a.R + i];
            tab[1][p][rl] = a.invk[p * a.N + ((i + a.off) ^ a.pxor)];
            tab[2][p][rl] = a.posdot[p * a.R + i];
            tab[3][p][rl] = a.qA[p * a.R + i];
            tab[4][p][rl] = a.qIYR[p * a.R + i];
        }
    for (int p = 0; p < P; ++p) {
        float ce = 0.f;
        const float negsum = fold_partials(a.rowpart, a.nJt, P, p, a.R, i, i < a.R, fold);
        if (mine) {
            const float neg = negsum;
            const float iq = tab[0][p][rl], ik = tab[1][p][rl], S = tab[2][p][rl], iqP = tab[0][P - 1][rl];
            const float x = fmaf(S * tab[3][p][rl], ik, a.cshift);
            const float epos = __builtin_amdgcn_exp2f(x);
            const float Z = neg + epos;
            ce = ce_from(neg, epos, x, Z);
            if (a.row_lse_out) a.row_lse_out[p * a.R + i] = logf(Z) + a.lse_offset;
            if (a.pos_logit_out) a.pos_logit_out[p * a.R + i] = a.scale * S * iq * ik + a.bias;
            const float invZ = 1.0f / Z;
            a.negfrac[p * a.R + i] = neg * invZ;
            // band-operand scale: beta_p / gam = sgn w_p inv_p / inv_P (folded into the exponent)
            a.qC[p * a.R + i] = a.cshift + log2f(a.wnorm[p] * iq / iqP);
            a.qRho[p * a.R + i] = a.sgn * invZ;
            a.qKap[p * a.R + i] = a.sgn * invZ * tab[4][p][rl];
            if (a.kind == kRows) a.diagA[p * a.R + i] = -a.wnorm[p] * a.scale * (neg * invZ) * a.inv_den * iq * ik;
        }
        lead_sum_write(ce, &a.lossparts[((int64_t)a.slot0 + blockIdx.x) * P + p]);
    }
}

__global__ __launch_bounds__(64 * kStatWaves, 8) void k_colstats(StatsArgs a) {  // two blocks per CU
    __shared__ float fold[kStatWaves][kStatRows];
    __shared__ float tab[5][kMaxP][kStatRows];  // inv_k, kIYR, inv_q and posdot * qA of the positive, row negfrac
    const int rl = threadIdx.x % kStatRows;
    const int64_t j = (int64_t)blockIdx.x * kStatRows + rl;
    const bool lead = threadIdx.x < kStatRows;
    const bool mine = lead && j < a.N;
    const int P = a.pf.n;
    const int64_t i = j - a.off;  // the query row whose positive is column j, if any
    const bool haspos = mine && i >= 0 && i < a.R;
    const bool sym = a.kind == kInfonce;
    if (mine)
        for (int p = 0; p < P; ++p) {
            tab[0][p][rl] = a.invk[p * a.N + j];
            tab[1][p][rl] = a.kIYR[p * a.N + j];
            tab[2][p][rl] = haspos ? a.invq[p * a.R + i] : 0.f;
            tab[3][p][rl] = haspos ? a.posdot[p * a.R + i] * a.qA[p * a.R + i] : 0.f;
            tab[4][p][rl] = sym ? a.negfrac[p * a.R + j] : 0.f;
        }
    for (int p = 0; p < P; ++p) {
        float ce = 0.f;
        const float negsum = fold_partials(a.colpart, a.nIt, P, p, a.N, j, j < a.N, fold);
        if (mine) {
            const float neg = negsum;
            const float ik = tab[0][p][rl], ikP = tab[0][P - 1][rl];
            float epos = 0.f, x = 0.f;
            if (haspos) {
                x = fmaf(tab[3][p][rl], ik, a.cshift);
                epos = __builtin_amdgcn_exp2f(x);
            }
            const float Z = neg + epos;
            if (a.col_lse_out) a.col_lse_out[p * a.N + j] = logf(Z) + a.lse_offset;
            a.kC[p * a.N + j] = a.cshift + log2f(a.wnorm[p] * ik / ikP);
            if (sym) {
                const float invZ = 1.0f / Z;
                ce = ce_from(neg, epos, x, Z);
                a.kNegfrac[p * a.N + j] = neg * invZ;
                a.kRho[p * a.N + j] = a.sgn * invZ;
                a.kKap[p * a.N + j] = a.sgn * invZ * tab[1][p][rl];
                // positive cell (j, j): g = -(neg_r / Z_r + neg_c / Z_c) / 2N
                a.diagA[p * a.R + j] =
                    -a.wnorm[p] * a.scale * (tab[4][p][rl] + neg * invZ) * a.inv_den * tab[2][p][rl] * ik;
            } else {
                a.kRho[p * a.N + j] = 0.f;
                a.kKap[p * a.N + j] = 0.f;
                a.kNegfrac[p * a.N + j] = 0.f;
            }
        }
        lead_sum_write(ce, &a.lossparts[((int64_t)a.slot0 + blockIdx.x) * P + p]);
    }
}

// SigLIP tables (one thread per query row, then per key row) and the
// positive cells' loss and gradient coefficients.
__global__ __launch_bounds__(256) void k_siglip_tabs(StatsArgs a) {
    __shared__ float red[4];
    const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int P = a.pf.n;
    for (int p = 0; p < P; ++p) {
        float lpos = 0.f, sig_neg = 0.f;
        if (r < a.R) {
            const int64_t i = r;
            const float iq = a.invq[p * a.R + i], ik = a.invk[p * a.N + ((i + a.off) ^ a.pxor)];
            a.qC[p * a.R + i] = a.sgn * a.wnorm[p] * iq / a.invq[(P - 1) * a.R + i];
            if (a.nopos) {  // no implicit positive: its loss, residual and coefficient are 0
                a.diagA[p * a.R + i] = 0.f;
            } else {
                const float S = a.posdot[p * a.R + i];
                const float l = a.scale * S * iq * ik + a.bias;
                // softplus(-l) and sigmoid(-l), both overflow-free
                const float t = expf(-fabsf(l));
                lpos = fmaxf(-l, 0.f) + log1pf(t);
                sig_neg = (l >= 0.f) ? t / (1.f + t) : 1.f / (1.f + t);
                a.diagA[p * a.R + i] = -a.mirror * a.wnorm[p] * a.scale * sig_neg * a.inv_den * iq * ik;
                if (a.pos_logit_out) a.pos_logit_out[p * a.R + i] = l;
            }
        } else if (r < a.R + a.N) {
            const int64_t j = r - a.R;
            const float ik = a.invk[p * a.N + j];
            a.kC[p * a.N + j] = a.sgn * a.wnorm[p] * ik / a.invk[(P - 1) * a.N + j];
        }
        block_sum_write(lpos, red, &a.lossparts[((int64_t)a.slot0 + blockIdx.x) * P + p]);
        // the positive cell's residual is sigma(l) - 1 = -sigma(-l)
        if (a.biasparts) block_sum_write(-sig_neg, red, &a.biasparts[((int64_t)a.slot0 + blockIdx.x) * P + p]);
    }
}

// ----------------------------------------------------------------------------
// k_bwd: one pass of the backward (row pass or column pass).
//
// Workgroup = 64 outer rows (the rows whose gradient the pass owns), 4 waves,
// one per SIMD; wave w owns the w-th quarter of the prefix width Dw, both for
// the logit recompute and for the gradient, so every inner element it reads
// from LDS feeds four MFMAs and is read by one wave only.  The outer rows'
// quarter stays in registers as FP16 MFMA operands for the whole pass, the
// gradient quarter (64 x Dw/4) in FP32 accumulators.  For every block of 16
// inner rows (one FP16 row-major tile in LDS, copied global->LDS two blocks
// ahead into a ring of three):
//  R: each wave forms its partial S^T over its quarter (16x16x32 FP16 MFMA)
//     and stores it, plus snapshots at prefix ends inside the quarter, to
//     LDS slots; S^p is the sum of the quarters below P_p plus the snapshot.
//  E: lane o of wave w forms, for outer row o and inner rows 4w..4w+3, the
//     cell coefficients a^p = dL/dS^p with every scale folded in (softmax:
//     2^{S A_o iy_n + C_o} (Rho_o iy_n + Kap_n); sigmoid: sigma(l) Bt_o iy_n),
//     the radial sums C^p_o += a^p S^p, and the band operands
//     A_b = sum_{p>=b} a^p (suffix sums, widest band first), stored in FP16.
//  U: dX[:, quarter] += A_band . Y[:, quarter] with 32x32x16 FP16 MFMA; the
//     inner tile is read transposed (ds_read_b64_tr_b16), so one copy serves
//     both contractions.
// Operands are exact power-of-two rescalings: inner and outer rows by their
// sig (BF16 -> FP16 is exact in range), and every outer row's band operand by
// a static scale fixed before the pass from an upper bound of |A_1| over all
// inner rows (the statistics bound every probability by the row's and the
// column's negative mass), so FP16 operands stay below 2^14; the scale is
// folded into the row's exponent (or beta) term and divided out at the write.
// The positive cell is left out; the finalize kernel adds its exact FP32 term.
// Barriers wait for LDS only: each wave waits for its own copies explicitly,
// so the copies of the next blocks stay in flight across barriers.
// ----------------------------------------------------------------------------
constexpr int BO = 64;
constexpr int BI = 16;
constexpr int NYBUF = 3;    // inner tiles in flight
constexpr int SLOTP = 20;   // floats per outer row of an S slot (16 + 4: conflict-free 16-byte accesses)
constexpr int APITCH = 24;  // FP16 per outer row of a band operand (16 + 8: conflict-free 16-byte reads)

template <uint32_t MASK>
struct Ladder {
    static constexpr int NP = __builtin_popcount(MASK);
    static constexpr int NDS = 32 - __builtin_clz(MASK);  // 32-wide steps of the widest prefix
    static constexpr int NQ = NDS / 4;                    // 32-wide steps per wave quarter
    static constexpr int DW = 32 * NDS;
    static constexpr int YP = DW + 16;                    // FP16 per LDS row of an inner tile
    static constexpr int end(int p) {                     // steps covered by prefix p
        int c = -1;
        for (int ds = 0; ds < 32; ++ds)
            if (MASK & (1u << ds)) {
                ++c;
                if (c == p) return ds + 1;
            }
        return -1;
    }
    // prefixes that end strictly inside a wave's quarter need a snapshot slot
    static constexpr uint32_t interior() {
        uint32_t m = 0;
        for (int p = 0; p < NP; ++p)
            if (end(p) % NQ != 0) m |= 1u << (end(p) - 1);
        return m;
    }
    static constexpr uint32_t INT_MASK = interior();
    static constexpr int NSLOT = 4 + __builtin_popcount(INT_MASK);
    // local steps (within a quarter) after which some wave takes a snapshot
    static constexpr uint32_t local_snaps() {
        uint32_t m = 0;
        for (int J = 0; J < NDS; ++J)
            if (INT_MASK & (1u << J)) m |= 1u << (J % NQ);
        return m;
    }
    static constexpr uint32_t LPOS = local_snaps();
    // local steps at which the band of some wave's 32-wide output block changes (step 0 always)
    static constexpr int band_at(int J) { return __builtin_popcount(MASK & ((1u << J) - 1u)); }
    static constexpr uint32_t band_steps() {
        uint32_t m = 1u;
        for (int J = 1; J < NDS; ++J)
            if (J % NQ != 0 && band_at(J) != band_at(J - 1)) m |= 1u << (J % NQ);
        return m;
    }
    static constexpr uint32_t BAND_STEPS = band_steps();
    static constexpr int wave_of(int p) { return (end(p) - 1) / NQ; }
    static constexpr int snap_slot(int p) {  // slot holding S^p's last quarter
        return (end(p) % NQ == 0) ? wave_of(p) : 4 + __builtin_popcount(INT_MASK & ((1u << (end(p) - 1)) - 1));
    }
};



typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;

__device__ __forceinline__ f16x4 ds_read_tr(const _Float16 *p) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p);
    return __builtin_bit_cast(f16x4, v);
}

// The finalize terms applied in place when a pass has one inner split: the radial sums C^p
// of the 64 rows (four waves' parts, fixed order), the positive cell's exact FP32 term and
// the normalisation Jacobian's radial part, then the finished gradient rows (zeros beyond
// the widest prefix).  The same arithmetic as k_finalize with nsplit = 1.
template <int NP, int NQ, uint32_t MASK>
__device__ __forceinline__ void bwd_finish(const BwdArgs &a, const f32x16 (&dacc)[2][NQ], const float (&Cacc)[NP],
                                        float csc, float *red, const float *inv_sc, int o0, int w, int lane,
                                        int tid) {
    constexpr int DW = 32 * (32 - __builtin_clz(MASK));
    const int NO = (int)a.NO, D = a.D;
    const int l32 = lane & 31, h32 = lane >> 5;
    lds_barrier();
    float *fin = red + 4 * NP * BO;  // [2][NP][BO]: running DG and RD per band
#pragma unroll
    for (int p = 0; p < NP; ++p) red[(w * NP + p) * BO + lane] = Cacc[p];
    lds_barrier();
    if (w == 0) {
        const int o = o0 + lane;
        float dg = 0.f, rd = 0.f, ts = 0.f;
        if (o < NO) {
            const int64_t ipos = o + a.pos_shift;
            const bool has_pos = ipos >= 0 && ipos < a.R;
            const float g = a.gam[o];
#pragma unroll
            for (int p = NP - 1; p >= 0; --p) {
                const float c = (((red[(0 * NP + p) * BO + lane] + red[(1 * NP + p) * BO + lane]) +
                                  red[(2 * NP + p) * BO + lane]) + red[(3 * NP + p) * BO + lane]) * csc;
                const float dA = has_pos ? a.diagA[p * a.R + ipos] : 0.f;
                const float dS = has_pos ? a.posdot[p * a.R + ipos] : 0.f;
                const float ix = a.invx[p * a.NO + o];
                const float T = fmaf(dA, dS, c * g);  // (w_p / W) s sum_j g_oj cos_oj
                dg += dA;
                rd += ix * ix * T;
                ts += T;
                fin[p * BO + lane] = dg;
                fin[(NP + p) * BO + lane] = rd;
            }
            if (a.tsum) a.tsum[o] = ts;
        }
    }
    lds_barrier();
    // per (block of 32 columns, 32 rows): the 16 rows' x and positive-row y first, then the rows
    const u16 *__restrict__ fx = a.finX;
    const u16 *__restrict__ fy = a.finY;
    float *__restrict__ out = a.fin_out;
    const bool accumulate = a.accumulate != 0;
#pragma unroll
    for (int ob = 0; ob < 2; ++ob) {
        float sc[16];
        int64_t xoff[16], yoff[16];
        bool ok[16], pos[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int orow = ob * 32 + 8 * (r >> 2) + 4 * h32 + (r & 3);
            const int o = o0 + orow;
            ok[r] = o < NO;
            const int64_t ipos = o + a.pos_shift;
            pos[r] = ok[r] && ipos >= 0 && ipos < a.R;
            sc[r] = ok[r] ? inv_sc[orow] * a.gam[o] : 0.f;
            xoff[r] = (int64_t)(ok[r] ? o : 0) * D;
            yoff[r] = pos[r] ? (int64_t)((o + a.diag_shift) ^ a.pxor) * D : 0;
        }
#pragma unroll
        for (int jb = 0; jb < NQ; ++jb) {
            const int d = w * (DW / 4) + 32 * jb + l32;
            const int band = __builtin_popcount(MASK & ((1u << (w * NQ + jb)) - 1u));
            float xv[16], yv[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                xv[r] = __uint_as_float((unsigned int)fx[xoff[r] + d] << 16);
                yv[r] = pos[r] ? __uint_as_float((unsigned int)fy[yoff[r] + d] << 16) : 0.f;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int orow = ob * 32 + 8 * (r >> 2) + 4 * h32 + (r & 3);
                const float v = fmaf(fin[band * BO + orow], yv[r],
                                     fmaf(-fin[(NP + band) * BO + orow], xv[r], dacc[ob][jb][r] * sc[r]));
                if (ok[r]) {
                    float *p = out + xoff[r] + d;
                    *p = accumulate ? *p + v : v;
                }
            }
        }
    }
    if (DW < D && !a.accumulate) {
        for (int e = tid; e < BO * (D - DW); e += 256) {
            const int orow = e / (D - DW), d = DW + e % (D - DW);
            if (o0 + orow < NO) a.fin_out[(int64_t)(o0 + orow) * D + d] = 0.f;
        }
    }
}

// SIG: sigmoid form; UPD: the gradient contraction runs; LOSS: the pass also sums the sigmoid
// form's loss; BIAS: and sigma(l) for dL/dbias; LIST: listed cells (extra positives) are left
// out of the pass.  Compile-time choices, so the epilogue has no branch and carries only the
// sums a call asks for.
template <uint32_t MASK, bool SIG, bool UPD, bool LOSS, bool BIAS, bool LIST>
__global__ __launch_bounds__(256, 1) void k_bwd(BwdArgs a) {
    using L = Ladder<MASK>;
    constexpr int NP = L::NP;
    constexpr int NQ = L::NQ;
    constexpr int DW = L::DW;
    constexpr int YP = L::YP;
    constexpr int NSLOT = L::NSLOT;
    constexpr int RPW = BI / 4;                // inner rows this wave copies per block
    constexpr int IPR = (DW / 8 + 63) / 64;    // 1 KB pieces per inner row
    constexpr bool FULLP = (DW / 8) % 64 == 0;  // every lane of every piece active
    constexpr int NCW = RPW * IPR;             // row copy instructions per wave per block
    static_assert(NQ >= 1 && L::NDS % 4 == 0, "the widest prefix must be a multiple of 128");
    static_assert(IPR == 1 || (FULLP && IPR == 2), "an inner row is one partial or one or two whole 1 KB pieces");

    constexpr int RSL = BI * YP + 512;  // FP16 elements per ring slot: the tile, then its tables [iI | iKap][p][row]
    __shared__ __attribute__((aligned(16))) _Float16 Ys[NYBUF][RSL];
    __shared__ __attribute__((aligned(16))) float Sl[NSLOT][BO * SLOTP];
    __shared__ __attribute__((aligned(16))) _Float16 At[NP][BO * APITCH];
    __shared__ float inv_sc[BO];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4, l32 = lane & 31, h32 = lane >> 5;
    const int NO = (int)a.NO, NI = (int)a.NI, dsh = (int)a.diag_shift;
    const int o0 = (int)blockIdx.x * BO;
    const int o = o0 + lane;  // the outer row of this lane in the E-phase
    const bool ovalid = o < NO;
    const int nblocks = (NI + BI - 1) / BI;
    const int nb_begin = (int)blockIdx.y * (int)a.blocks_per_split;
    const int nb_end = min(nb_begin + (int)a.blocks_per_split, nblocks);
    const int D = a.D;
    const int dq0 = w * (DW / 4);  // first column of this wave's quarter

    // ---- this lane's outer-row terms (every wave holds the same 64 rows)
    float Ao[NP], Co[NP], Ro[NP];
    float csc = 1.0f;  // 1 / (static scale * sig) of this lane's row, for the radial sums
    {
        const int64_t orow = ovalid ? o : 0;
        float sc = 1.0f;
        if (ovalid) {
            const float ixP = a.oInv[(NP - 1) * a.NO + orow];
            float U = 0.f;
            for (int p = 0; p < NP; ++p) {
                const float own = a.oNeg ? a.oNeg[p * a.NO + orow] : 0.f;
                const float gt = a.gterm ? a.gterm[p] : a.gterm_val[p];
                U += a.wnorm[p] * (a.oInv[p * a.NO + orow] / ixP) * a.iyrmax[p] * (own + gt);
            }
            if (U > 0.f) sc = ldexpf(1.0f, max(-126, min(126, 14 - (ilogbf(U) + 1))));
        }
        const float rsig = 1.0f / a.oSig[orow];  // exact: sig is a power of two
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            Ao[p] = a.oA[p * a.NO + orow] * rsig;
            const float c = a.oC[p * a.NO + orow];
            Co[p] = SIG ? c * sc : c + log2f(sc);
            Ro[p] = SIG ? 0.f : a.oRho[p * a.NO + orow];
        }
        csc = rsig / sc;
        if (w == 0) inv_sc[lane] = 1.0f / sc;
    }

    // ---- copies of an inner block into a ring slot.  This wave copies inner rows
    // 4 w .. 4 w + 3 (the FP16 inner matrix carries two zero blocks past its last row,
    // so no row index is clamped) and one float of the block's tables per lane.
    uint32_t cvo[RPW];  // this lane's byte offset in each of its rows, from the block start
#pragma unroll
    for (int k = 0; k < RPW; ++k) cvo[k] = (uint32_t)(4 * w + k) * (uint32_t)D * 2u + 16u * (uint32_t)lane;
    // ring slots are addressed by byte offsets from the first slot; LDS addresses of this
    // wave's rows and table entries within a slot (wave-uniform)
    const uint32_t ys_lds = (uint32_t)(uintptr_t)&Ys[0][0];
    uint32_t rowb[RPW];
#pragma unroll
    for (int k = 0; k < RPW; ++k) rowb[k] = __builtin_amdgcn_readfirstlane(ys_lds + 2u * (uint32_t)((4 * w + k) * YP));
    const uint32_t tabb = __builtin_amdgcn_readfirstlane(ys_lds + 2u * (uint32_t)(BI * YP) + 4u * (uint32_t)(64 * w));
    auto copy_row = [&](const _Float16 *gblk, uint32_t ybb, auto kc) {  // row 4 w + k of the block at gblk into slot ybb
        constexpr int k = decltype(kc)::value;
        if constexpr (IPR == 2)
            dma_row2_add(gblk, cvo[k], ybb, rowb[k]);
        else if constexpr (FULLP)
            dma_row1_add(gblk, cvo[k], ybb, rowb[k]);
        else if (lane < DW / 8)
            dma_row1_add(gblk, cvo[k], ybb, rowb[k]);
    };
    // table entry [which][p][r] of this lane (lanes past the end copy a harmless float)
    const int te = 64 * w + lane;
    const bool tact = te < 2 * NP * BI;
    const int tr = te % BI;
    const float *tbase = tact ? ((te / (NP * BI)) == 0 ? a.iI : a.iKap) + (int64_t)((te / BI) % NP) * NI + tr : a.iI;
    const int tlim = tact ? NI - 1 - tr : 0;  // rows past the end read the last row
    auto copy_tables = [&](int nb, uint32_t ybb) { dma4_add(tbase + min(nb * BI, tlim), ybb, tabb); };
    const _Float16 *gcp = a.Y16 + (int64_t)nb_begin * BI * D;  // the next block to copy
    auto issue_block = [&](int nb, uint32_t ybb) {
        static_for<0, RPW>([&](auto kc) { copy_row(gcp, ybb, kc); });
        copy_tables(nb, ybb);
        gcp += (int64_t)BI * D;
    };

    // zero the ring once so that every LDS word the kernel reads was written
    for (int e = tid; e < NYBUF * RSL / 8; e += 256) *(uint4 *)&Ys[0][e * 8] = make_uint4(0, 0, 0, 0);
    lds_barrier();

    // ---- outer rows' quarter as B operands: rows 16 ob + l16, columns dq0 + 32 ks + 8 g4
    f16x8 xr[4][NQ];
#pragma unroll
    for (int ob = 0; ob < 4; ++ob) {
        const int64_t orow = o0 + 16 * ob + l16;
        const _Float16 *src = a.X16 + (orow < a.NO ? orow : 0) * D + dq0 + 8 * g4;
#pragma unroll
        for (int ks = 0; ks < NQ; ++ks) {
            f16x8 v = {};
            if (orow < a.NO) v = *(const f16x8 *)(src + 32 * ks);
            xr[ob][ks] = v;
        }
    }

    f32x16 dacc[2][NQ];
#pragma unroll
    for (int ob = 0; ob < 2; ++ob)
#pragma unroll
        for (int j = 0; j < NQ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) dacc[ob][j][r] = 0.f;
    float Cacc[NP], Lacc[NP], Bacc[NP];  // radial sums; sigmoid form: loss and sum of sigma(l)
#pragma unroll
    for (int p = 0; p < NP; ++p) Cacc[p] = Lacc[p] = Bacc[p] = 0.f;

    // ---- Two-phase software pipeline.  Epilogue E of a block = one unit per prefix
    // (lane = outer row, inner rows 4 w .. 4 w + 3, four independent chains), widest
    // prefix first so that the band operand A_p = sum_{p' >= p} a^p' is a running sum.
    // Its NA widest units (E_a) run in phase B beside the update MFMAs of the block
    // before; the rest (E_b) in phase A beside the recompute MFMAs of the block after:
    //   phase A(t): recompute of t + 1 | E_b(t) | copies of t + 2      -> barrier
    //   phase B(t): update of t         | E_a(t + 1)                   -> barrier
    // E_a's band operands are held in registers until phase A writes them, because
    // the update of t reads the band operand buffer during phase B.
    // prefixes NP - NA .. NP - 1 belong to E_a.  Measured: on ladders of four or more prefixes the
    // softmax form runs every unit beside the recompute and the update alone; on ladders of five or
    // more the sigmoid form puts three units beside the update in its pass with the loss and one in
    // the pass without (an even split makes its live values outgrow the register file, and the
    // outer-row operands are then reloaded from scratch inside the loop).  Otherwise an even split.
    constexpr int NA = SIG ? (NP >= 5 ? (LOSS ? 3 : 1) : NP / 2) : (NP >= 4 ? 0 : NP / 2);
    f32x4 sv[NSLOT];
    auto read_slots = [&]() {
#pragma unroll
        for (int s = 0; s < NSLOT; ++s) sv[s] = *(const f32x4 *)&Sl[s][lane * SLOTP + 4 * w];
    };
    float run[4] = {0.f, 0.f, 0.f, 0.f};
    f16x4 hv[NA > 0 ? NA : 1];
    // blocks whose cells need masks: from nb_sp on (ragged or past the split's end; every
    // block if the outer rows are ragged), and those holding positives of these outer rows
    const int nb_sp = o0 + BO > NO ? 0 : min(NI / BI, nb_end);
    // blocks with c_lo < n0 < c_lo + BO + BI hold positives (one-set form: and the cells of a row
    // with itself; a pair's two rows are adjacent, so the range grows by one row on either side)
    const int pxr = a.pxor;
    const int c_lo = o0 + dsh - BI - pxr;
    const uint32_t c_len = (uint32_t)(BO + BI - 1 + 2 * pxr);
    // listed cells (extra positives): this outer block's entries, sorted by nb; lnb is the nb of
    // entry lcur (INT_MAX past the last).  Blocks are visited in increasing order, so the cursor
    // only moves forward, and it reads an entry only when it passes one.
    // (LIST: a compile-time variant, so that calls without lists keep the plain block loop.)
    int lcur = 0, lend = 0;
    if constexpr (LIST) {
        lcur = a.lptr[blockIdx.x];
        lend = a.lptr[blockIdx.x + 1];
    }
    int lnb = LIST && lcur < lend ? a.lent[lcur].nb : INT_MAX;
    auto listed = [&](int nb) {
        if constexpr (!LIST) return false;
        while (lnb < nb) {
            ++lcur;
            lnb = lcur < lend ? a.lent[lcur].nb : INT_MAX;
        }
        return lnb == nb;
    };
    auto needmask = [&](int nb) { return nb >= nb_sp || (uint32_t)(nb * BI - c_lo - 1) < c_len || listed(nb); };
    // lane masks of block nb's cells for inner rows 4 w + t (wave-uniform 64-bit masks)
    const uint64_t ovm = __builtin_amdgcn_ballot_w64(ovalid);
    auto block_masks = [&](int nb, uint64_t(&mk)[4]) {
        if (!needmask(nb)) {
#pragma unroll
            for (int t = 0; t < 4; ++t) mk[t] = ovm;
        } else {
            const int nw = nb * BI + 4 * w;
            const int lim = min(NI, nb_end * BI);
#pragma unroll
            for (int t = 0; t < 4; ++t)
                mk[t] = __builtin_amdgcn_ballot_w64(ovalid && nw + t < lim && nw + t != ((o + dsh) ^ pxr) &&
                                                    (pxr == 0 || nw + t != o + dsh));
            if (listed(nb)) {
                const uint64_t *lm = a.lent[lcur].m + 4 * w;
#pragma unroll
                for (int t = 0; t < 4; ++t) mk[t] &= ~lm[t];
            }
        }
    };
    // Epilogue unit of prefix p for the block in ring slot eyo (its tables follow the tile): the
    // table reads (utab) and four parts that the phases spread over their MFMA steps, one or two
    // per step: (0) S^p and S^p A_o, (1) the logits and exponentials, (2) the coefficients,
    // (3) the running band operand, the radial sums and the FP16 band operand.
    const char *tabs0 = (const char *)&Ys[0][BI * YP] + 16 * w;  // this wave's four inner rows
    struct UTab {
        f32x4 iy, kp;
    };
    auto utab = [&](auto pc, uint32_t eyb) {
        constexpr int p = decltype(pc)::value;
        UTab tb;
        tb.iy = *(const f32x4 *)(tabs0 + eyb + 4 * p * BI);
        if constexpr (!SIG) tb.kp = *(const f32x4 *)(tabs0 + eyb + 4 * (NP + p) * BI);
        return tb;
    };
    struct UState {
        f32x4 Sp, e;
        float av[4];
    };
    auto upart = [&](auto pc, auto kc, auto masked, const uint64_t(&mk)[4], const UTab &tb, UState &st) {
        constexpr int p = decltype(pc)::value;
        constexpr int k = decltype(kc)::value;
        constexpr bool MK = decltype(masked)::value;
        if constexpr (k == 0) {
            // S^p: quarters below wave_of(p), lowest first (shared by the prefixes), plus the snapshot
            if constexpr (L::wave_of(p) == 0) {
                st.Sp = sv[L::snap_slot(p)];
            } else {
                st.Sp = sv[0];
                static_for<1, L::wave_of(p)>([&](auto qc) { st.Sp += sv[decltype(qc)::value]; });
                st.Sp += sv[L::snap_slot(p)];
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) st.e[t] = st.Sp[t] * Ao[p];
        } else if constexpr (k == 1) {
            if constexpr (!SIG) {
                // e = 2^(S A_o iy + C_o)
                float x[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) x[t] = fmaf(st.e[t], tb.iy[t], Co[p]);
#pragma unroll
                for (int t = 0; t < 4; ++t) st.e[t] = __builtin_amdgcn_exp2f(x[t]);
            } else if constexpr (!LOSS) {
                // the unmasked coefficient sigma(l) beta_o iy; sigma = 1 / (1 + 2^-u) directly (2^-u = inf
                // gives 0), with no loss term to share 2^-|u| with
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float uu = fmaf(st.e[t], tb.iy[t], a.b2);
                    const float sg = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-uu));
                    st.e[t] = sg * Co[p] * tb.iy[t];  // Co holds beta_o for the sigmoid form
                }
            } else {
                // the unmasked coefficient sigma(l) beta_o iy, and the loss: softplus(l) / ln 2 =
                // max(u, 0) + log2(1 + tt) per cell, the four cells' log2(1 + tt) taken as one
                // log2 of the product of their (1 + tt) (each in (1, 2]), each with log1p's rounding
                // corrected to first order
                float prod = 1.f, lsum = 0.f;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float uu = fmaf(st.e[t], tb.iy[t], a.b2);
                    const float tt = __builtin_amdgcn_exp2f(-fabsf(uu));
                    const float wq = 1.f + tt;
                    const float rr = __builtin_amdgcn_rcpf(wq);
                    const float sg = uu >= 0.f ? rr : tt * rr;
                    st.e[t] = sg * Co[p] * tb.iy[t];  // Co holds beta_o for the sigmoid form
                    if constexpr (LOSS) {
                        const float corr = (tt - (wq - 1.f)) * rr * kLog2e;
                        const bool in = !MK || __builtin_amdgcn_inverse_ballot_w64(mk[t]);
                        prod *= in ? wq : 1.f;
                        lsum += in ? fmaxf(uu, 0.f) + corr : 0.f;
                        if constexpr (BIAS) Bacc[p] += in ? sg : 0.f;  // sigma(l), unscaled
                    }
                }
                if constexpr (LOSS) Lacc[p] += __builtin_amdgcn_logf(prod) + lsum;
            }
        } else if constexpr (k == 2) {
            // a^p = e (Rho_o iy + Kap) (softmax) or e (sigmoid), masked
#pragma unroll
            for (int t = 0; t < 4; ++t) st.av[t] = SIG ? st.e[t] : st.e[t] * fmaf(Ro[p], tb.iy[t], tb.kp[t]);
            if constexpr (MK)
#pragma unroll
                for (int t = 0; t < 4; ++t) st.av[t] = __builtin_amdgcn_inverse_ballot_w64(mk[t]) ? st.av[t] : 0.f;
        } else {
            // band operand suffix sums, radial sums, FP16 band operand
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if constexpr (p == NP - 1)
                    run[t] = st.av[t];
                else
                    run[t] += st.av[t];
            }
            Cacc[p] = fmaf(st.av[0], st.Sp[0],
                           fmaf(st.av[1], st.Sp[1], fmaf(st.av[2], st.Sp[2], fmaf(st.av[3], st.Sp[3], Cacc[p]))));
            if constexpr (UPD) {
                // two values per conversion (round to nearest even), instead of a fused multiply-add per value
                uint32_t h01, h23;
                asm("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(h01) : "v"(run[0]), "v"(run[1]));
                asm("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(h23) : "v"(run[2]), "v"(run[3]));
                const f16x4 v = __builtin_bit_cast(f16x4, (uint64_t)h01 | ((uint64_t)h23 << 32));
                if constexpr (p >= NP - NA)
                    hv[NP - 1 - p] = v;  // E_a: held until phase A
                else
                    *(f16x4 *)&At[p][lane * APITCH + 4 * w] = v;
            }
        }
    };
    // Schedules (compile time): the step of part k of unit u and of its table reads.  Phase A
    // runs E_b (units u = 0 .. NUB - 1 are prefixes NUB - 1 - u), phase B runs E_a (units
    // u = 0 .. NA - 1 are prefixes NP - 1 - u) from its second step on (the S slots are read
    // just before it); a table step of -1 is before the first step.
    constexpr int NUB = NP - NA;
    struct Sched {
        static constexpr int part_a(int u, int k) { return NUB > 0 ? ((4 * u + k) * NQ) / (4 * NUB) : 0; }
        static constexpr int tab_a(int u) { return part_a(u, 0) - 1; }
        static constexpr int part_b(int u, int k) {
            return NA > 0 ? (((4 * u + k) * (NQ - 1)) / (4 * NA) + 1 < NQ ? ((4 * u + k) * (NQ - 1)) / (4 * NA) + 1 : NQ - 1) : 0;
        }
        static constexpr int tab_b(int u) { return part_b(u, 0) - 1; }
    };

    // transposed inner-tile operands of the update, two steps ahead; the first two are
    // read before the barrier that publishes the band operands (the tile is stable)
    f16x8 bf[3];
    // per-lane part of the transposed reads (loop invariant); ring slot and step are immediates
    const _Float16 *ytr = &Ys[0][0] + (8 * ((lane >> 4) >> 1) + ((lane & 15) >> 2)) * YP + 16 * ((lane >> 4) & 1) +
                          4 * (lane & 3) + 32 * w * NQ;
    auto load_b = [&](uint32_t uyb, auto jc) {
        constexpr int jb = decltype(jc)::value;
        const _Float16 *ysrc = (const _Float16 *)((const char *)ytr + uyb) + 32 * jb;
        const f16x4 lo = ds_read_tr(ysrc);
        const f16x4 hi = ds_read_tr(ysrc + 4 * YP);
        bf[jb % 3] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    auto u_pre = [&](uint32_t uyb) {
        load_b(uyb, std::integral_constant<int, 0>{});
        if constexpr (NQ > 1) load_b(uyb, std::integral_constant<int, 1>{});
    };
    // phase A: recompute of the tile in ring slot rbuf (partial S^T over this wave's quarter,
    // 16 inner x 64 outer, into the S slots) | E_b of block nb (tables in ebuf) | copies of
    // block cnb into cbuf, each spread over the recompute steps
    auto phase_a = [&](auto masked, auto with_e, uint32_t ryo, int nb, uint32_t eyo, int cnb, uint32_t cyo) {
        constexpr bool WE = decltype(with_e)::value;
        uint64_t mk[4];
        if constexpr (decltype(masked)::value) block_masks(nb, mk);
        f32x4 acc[4];
#pragma unroll
        for (int ob = 0; ob < 4; ++ob) acc[ob] = f32x4{0.f, 0.f, 0.f, 0.f};
        const _Float16 *yrow = (const _Float16 *)((const char *)&Ys[0][0] + ryo) + l16 * YP + dq0 + 8 * g4;
        auto put = [&](int slot) {
#pragma unroll
            for (int ob = 0; ob < 4; ++ob) *(f32x4 *)&Sl[slot][(16 * ob + l16) * SLOTP + 4 * g4] = acc[ob];
        };
        if constexpr (WE) {
            if constexpr (UPD)
                static_for<0, NA>([&](auto ic) {
                    constexpr int p = NP - 1 - decltype(ic)::value;
                    *(f16x4 *)&At[p][lane * APITCH + 4 * w] = hv[decltype(ic)::value];
                });
        }
        UTab tb[NUB > 0 ? NUB : 1];
        UState us[NUB > 0 ? NUB : 1];
        if constexpr (WE)
            static_for<0, NUB>([&](auto uc) {
                constexpr int u = decltype(uc)::value;
                if constexpr (Sched::tab_a(u) < 0) tb[u] = utab(std::integral_constant<int, NUB - 1 - u>{}, eyo);
            });
        f16x8 yv[2];
        yv[0] = *(const f16x8 *)yrow;
        static_for<0, NQ>([&](auto kc) {
            constexpr int ks = decltype(kc)::value;
            if constexpr (ks + 1 < NQ) yv[(ks + 1) & 1] = *(const f16x8 *)(yrow + 32 * (ks + 1));
            if constexpr (WE) {
                if constexpr (ks == 0) copy_tables(cnb, cyo);
                static_for<0, RPW>([&](auto kc) {
                    if constexpr ((decltype(kc)::value * NQ) / RPW == ks) copy_row(gcp, cyo, kc);
                });
            }
#pragma unroll
            for (int ob = 0; ob < 4; ++ob)
                acc[ob] = __builtin_amdgcn_mfma_f32_16x16x32_f16(yv[ks & 1], xr[ob][ks], acc[ob], 0, 0, 0);
            if constexpr (((L::LPOS >> ks) & 1u) != 0 && ks + 1 < NQ) {
                // waves with a prefix end at this step store a snapshot (a wave-uniform branch)
                const int J = w * NQ + ks;
                if ((L::INT_MASK >> J) & 1u) put(4 + __builtin_popcount(L::INT_MASK & ((1u << J) - 1u)));
            }
            if constexpr (WE)  // E_b units: prefixes NUB - 1 .. 0
                static_for<0, NUB>([&](auto uc) {
                    constexpr int u = decltype(uc)::value;
                    constexpr std::integral_constant<int, NUB - 1 - u> pc{};
                    static_for<0, 4>([&](auto kc) {
                        if constexpr (Sched::part_a(u, decltype(kc)::value) == ks) upart(pc, kc, masked, mk, tb[u], us[u]);
                    });
                    if constexpr (Sched::tab_a(u) == ks) tb[u] = utab(pc, eyo);
                });
            __builtin_amdgcn_sched_barrier(0);
        });
        put(w);
    };

    // phase B: dX[:, quarter] += A_band . Y[:, quarter] for the tile in ring slot ubuf | E_a of
    // block nb1 (tables in ebuf1).  The band operand is read only at the
    // steps where some wave's band changes (the same code for every wave, no branches).
    // (No branches in here: the gradient accumulators must not meet at a join.  E_a always
    // runs with masks; a block past the end has every cell masked.)
    auto phase_b = [&](auto with_u, uint32_t uyo, const uint64_t(&mk1)[4], uint32_t eyo1) {
        constexpr bool WE = NA > 0;
        constexpr bool WU = decltype(with_u)::value && UPD;
        constexpr std::true_type masked{};
        f16x8 af[2];
        UTab tb[NA > 0 ? NA : 1];
        UState us[NA > 0 ? NA : 1];
        if constexpr (WE)
            static_for<0, NA>([&](auto uc) {
                constexpr int u = decltype(uc)::value;
                if constexpr (Sched::tab_b(u) < 0) tb[u] = utab(std::integral_constant<int, NP - 1 - u>{}, eyo1);
            });
        static_for<0, NQ>([&](auto jc) {
            constexpr int jb = decltype(jc)::value;
            if constexpr (WU) {
                if constexpr ((L::BAND_STEPS >> jb) & 1u) {
                    const int band = __builtin_popcount(MASK & ((1u << (w * NQ + jb)) - 1u));
#pragma unroll
                    for (int ob = 0; ob < 2; ++ob)
                        af[ob] = *(const f16x8 *)&At[band][(32 * ob + l32) * APITCH + 8 * h32];
                }
                if constexpr (jb + 2 < NQ) load_b(uyo, std::integral_constant<int, jb + 2>{});
#pragma unroll
                for (int ob = 0; ob < 2; ++ob)
                    dacc[ob][jb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[ob], bf[jb % 3], dacc[ob][jb], 0, 0, 0);
            }
            if constexpr (WE)  // E_a units: prefixes NP - 1 .. NP - NA
                static_for<0, NA>([&](auto uc) {
                    constexpr int u = decltype(uc)::value;
                    constexpr std::integral_constant<int, NP - 1 - u> pc{};
                    static_for<0, 4>([&](auto kc) {
                        if constexpr (Sched::part_b(u, decltype(kc)::value) == jb) upart(pc, kc, masked, mk1, tb[u], us[u]);
                    });
                    if constexpr (Sched::tab_b(u) == jb) tb[u] = utab(pc, eyo1);
                });
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // ring slots (byte offsets) of blocks nb, nb + 1, nb + 2
    uint32_t yo0 = 0, yo1 = 2 * RSL, yo2 = 4 * RSL;  // bytes
    uint64_t mk1[4];  // lane masks of block nb + 1
    if (nb_begin < nb_end) {
        issue_block(nb_begin, yo0);
        issue_block(nb_begin + 1, yo1);  // past the split's end: rows of the next split or the zero blocks
        wait_vm_n<NCW + 1>();
        lds_barrier();  // block 0 visible
        phase_a(std::false_type{}, std::false_type{}, yo0, 0, 0, 0, 0);  // recompute of block 0 alone
        lds_barrier();  // slots of block 0 visible
        read_slots();
        block_masks(nb_begin, mk1);
        phase_b(std::false_type{}, 0, mk1, yo0);  // E_a of block 0 alone
    }

    for (int nb = nb_begin; nb < nb_end; ++nb) {
        wait_vm();      // block nb + 1 landed (issued a full block earlier)
        lds_barrier();  // slots of nb consumed, every wave past the update of nb - 1; block nb + 1 visible
        // phase A: recompute of nb + 1 (past the end: a block of zeros or of the next split) | E_b(nb) |
        // copies of nb + 2
        if (needmask(nb))
            phase_a(std::true_type{}, std::true_type{}, yo1, nb, yo0, nb + 2, yo2);
        else
            phase_a(std::false_type{}, std::true_type{}, yo1, nb, yo0, nb + 2, yo2);
        gcp += (int64_t)BI * D;
        block_masks(nb + 1, mk1);
        if constexpr (UPD) u_pre(yo0);
        lds_barrier();  // band operands of nb and slots of nb + 1 visible
        read_slots();
        phase_b(std::true_type{}, yo0, mk1, yo1);  // update of nb | E_a(nb + 1)
        const uint32_t y = yo0;
        yo0 = yo1, yo1 = yo2, yo2 = y;
    }

    // ---------------- write the raw gradient block (scale divided out) and the radial sums
    const int64_t split = blockIdx.y;
    if constexpr (UPD) {
        if (a.fin_out) {
            bwd_finish<NP, NQ, MASK>(a, dacc, Cacc, csc, &Sl[0][0], inv_sc, o0, w, lane, tid);
        } else {
            float *dst = a.part + split * a.NO * D;
#pragma unroll
            for (int ob = 0; ob < 2; ++ob)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int orow = ob * 32 + 8 * (r >> 2) + 4 * h32 + (r & 3);
                    const float s = inv_sc[orow];
                    if (o0 + orow < NO) {
                        float *rowp = dst + (int64_t)(o0 + orow) * D + dq0 + l32;
#pragma unroll
                        for (int jb = 0; jb < NQ; ++jb) rowp[32 * jb] = dacc[ob][jb][r] * s;
                    }
                }
        }
    }
    // radial sums and sigmoid loss: add the four waves' inner rows (slots are free now)
    lds_barrier();
    float *red = &Sl[0][0];  // [4][NP][BO], then [4][NP] twice
#pragma unroll
    for (int p = 0; p < NP; ++p) red[(w * NP + p) * BO + lane] = Cacc[p];
    if constexpr (SIG && LOSS) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const float v = wave_sum(Lacc[p]);
            const float u = wave_sum(Bacc[p]);
            if (lane == 0) {
                red[4 * NP * BO + w * NP + p] = v;
                red[4 * NP * BO + 4 * NP + w * NP + p] = u;
            }
        }
    }
    lds_barrier();
    if (w == 0 && ovalid && !(UPD && a.fin_out)) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const float c = ((red[(0 * NP + p) * BO + lane] + red[(1 * NP + p) * BO + lane]) +
                             red[(2 * NP + p) * BO + lane]) + red[(3 * NP + p) * BO + lane];
            a.Cpart[(split * NP + p) * a.NO + o] = c * csc;
        }
    }
    if (SIG && LOSS && tid < NP) {
        const float *lr = red + 4 * NP * BO;
        const float v = ((lr[0 * NP + tid] + lr[1 * NP + tid]) + lr[2 * NP + tid]) + lr[3 * NP + tid];
        const int64_t slot = (int64_t)a.loss_slot0 + split * gridDim.x + blockIdx.x;
        a.lossparts[slot * NP + tid] = v * kLn2;
        if constexpr (BIAS) {
            const float *br = lr + 4 * NP;
            a.biasparts[slot * NP + tid] = ((br[0 * NP + tid] + br[1 * NP + tid]) + br[2 * NP + tid]) + br[3 * NP + tid];
        }
    }
}

// ----------------------------------------------------------------------------
// k_bwd_gen: one backward pass (row or column) for any prefix ladder and widths up to 2048.
//
// The arithmetic of k_bwd (recompute of S over an inner block, cell coefficients with every
// scale folded in, band operands as running sums widest prefix first, dX += A_band . Y, the
// positive cell and the radial term left to k_finalize), laid out for generality: 32 outer rows
// per workgroup (a 2048-wide gradient quarter of 32 rows is 32 x 512 FP32 = 256 accumulators per
// lane), 4 waves, wave w owning the 32-wide steps [w NQ, (w + 1) NQ) of the recompute and of the
// update; prefix ends, snapshot slots and bands come from run-time tables; the phases of a block
// run one after another (recompute, barrier, epilogue, barrier, update, barrier) while the copies
// of the next block are in flight.  Lane l of the epilogue owns outer row l & 31 and inner rows
// 4 w + 2 (l >> 5) + {0, 1}.  Split partials always go to k_finalize.
// ----------------------------------------------------------------------------
constexpr int GBO = kGenOuter;

// Tile rows of a swizzled ring (SWZ) are unpadded and hold 16-byte chunk c of inner row r at
// chunk c ^ gen_swz(r): with this map both the recompute's 16-byte row reads and the update's
// transposed reads are free of bank conflicts (the padded pitch + 16 halves leaves the
// transposed reads at about 1.5x their conflict-free time).  It permutes chunks inside aligned
// groups of 16, so a swizzled ring needs rows whose copied width is a multiple of 128 halves.
__device__ __forceinline__ int gen_swz(int r) { return ((5 * (r & 3)) ^ (8 * ((r >> 2) & 1))) & 15; }

template <int NQ, bool SWZ = false>
struct GenLds {
    // FP16 per LDS row of an inner tile (unswizzled: + 16 keeps the recompute's 16-byte row reads
    // free of bank conflicts, + 8 left them and the transposed reads 2-way)
    static constexpr int YP = 4 * NQ * 32 + (SWZ ? 0 : 16);
    static constexpr int RSL = BI * YP + 2 * kMaxP * BI * 2;  // FP16 per ring slot: the tile, then its tables
    static constexpr int NSLOT = NQ >= 16 ? 7 : 12;           // S slots (4 wave partials + snapshots)
    static constexpr int NBAND = NQ >= 16 ? 7 : kMaxP + 1;    // band operands (prefixes, then a zero band)
};
int gen_max_slots(int nq) { return nq >= 16 ? GenLds<16>::NSLOT : GenLds<8>::NSLOT; }
int gen_max_bands(int nq) { return nq >= 16 ? GenLds<16>::NBAND : GenLds<8>::NBAND; }

typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;

// A ladder the generic backward can also take at compile time (LM: bit e set where a prefix ends at
// 32 (e + 1)), with the same slots as the host's tables: a prefix ending on its wave's last step
// uses that wave's partial, the others snapshot slots 4, 5, ... in prefix order.
template <uint64_t LM, int NQ>
struct GenLadder {
    static constexpr int P = __builtin_popcountll(LM);
    static constexpr int end_step(int p) {
        int c = -1;
        for (int e = 0; e < 64; ++e)
            if (((LM >> e) & 1ull) != 0ull && ++c == p) return e;
        return 0;
    }
    static constexpr int wave_of(int p) { return end_step(p) / NQ; }
    static constexpr int snap_slot(int p) {
        if ((end_step(p) + 1) % NQ == 0) return end_step(p) / NQ;
        int interior = 0;
        for (int q = 0; q < p; ++q)
            if ((end_step(q) + 1) % NQ != 0) ++interior;
        return 4 + interior;
    }
    // the snapshot slot written after step e (a prefix ending there, not on its wave's last
    // step), or -1
    static constexpr int snap_at(int e) {
        for (int p = 0; p < P; ++p)
            if (end_step(p) == e && (e + 1) % NQ != 0) return snap_slot(p);
        return -1;
    }
    // bit W set: wave W writes a snapshot after its step ks
    static constexpr uint32_t snap_waves(int ks) {
        uint32_t m = 0;
        for (int W = 0; W < 4; ++W)
            if (snap_at(W * NQ + ks) >= 0) m |= 1u << W;
        return m;
    }
    // the band operand of step j: the narrowest prefix that reaches past it (P: none, zero band)
    static constexpr int band_of(int j) {
        for (int p = 0; p < P; ++p)
            if (end_step(p) >= j) return p;
        return P;
    }
    // wave W's bands, 4 bits per step (NQ <= 16)
    static constexpr uint64_t bands(int W) {
        uint64_t m = 0;
        for (int jb = 0; jb < NQ; ++jb) m |= (uint64_t)band_of(W * NQ + jb) << (4 * jb);
        return m;
    }
};
// the Large and XL tiers' ladder {64, 128, 256, 512, 1024, 2048}
constexpr uint64_t kLadder2048 = (1ull << 1) | (1ull << 3) | (1ull << 7) | (1ull << 15) | (1ull << 31) | (1ull << 63);

template <int NQ, bool SIG, bool UPD, uint64_t LM = 0>
__global__ __launch_bounds__(256, 1) void k_bwd_gen(BwdArgs a) {
    // the compiled ladder (widest prefix 2048 = D) takes the swizzled ring, and its per-prefix
    // registers only for its own prefixes
    constexpr bool SWZ = LM != 0;
    constexpr int NPV = LM != 0 ? __builtin_popcountll(LM) : kMaxP;
    using G = GenLds<NQ, SWZ>;
    constexpr int YP = G::YP, RSL = G::RSL;
    __shared__ __attribute__((aligned(16))) _Float16 Ys[2][RSL];
    __shared__ __attribute__((aligned(16))) float Sl[G::NSLOT][GBO * SLOTP];
    __shared__ __attribute__((aligned(16))) _Float16 At[G::NBAND][GBO * APITCH];
    __shared__ float inv_sc[GBO];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4, l32 = lane & 31, h = lane >> 5;
    const int NO = (int)a.NO, NI = (int)a.NI, D = a.D, P = a.pf.n;
    const int o0 = (int)blockIdx.x * GBO;
    const int o = o0 + l32;  // this lane's outer row in the epilogue
    const bool ovalid = o < NO;
    const int nblocks = (NI + BI - 1) / BI;
    const int nb_begin = (int)blockIdx.y * (int)a.blocks_per_split;
    const int nb_end = min(nb_begin + (int)a.blocks_per_split, nblocks);
    const int dq0 = w * NQ * 32;  // first column of this wave's steps
    const int dsh = (int)a.diag_shift, pxr = a.pxor;
    const bool want_loss = SIG && a.want_loss != 0, want_bias = SIG && a.biasparts != nullptr;

    // ---- this lane's outer-row terms (the static operand scale as in k_bwd)
    float Ao[NPV], Co[NPV], Ro[NPV];
    float csc = 1.0f;
    {
        const int64_t orow = ovalid ? o : 0;
        float sc = 1.0f;
        if (ovalid) {
            const float ixP = a.oInv[(P - 1) * a.NO + orow];
            float U = 0.f;
            for (int p = 0; p < P; ++p) {
                const float own = a.oNeg ? a.oNeg[p * a.NO + orow] : 0.f;
                const float gt = a.gterm ? a.gterm[p] : a.gterm_val[p];
                U += a.wnorm[p] * (a.oInv[p * a.NO + orow] / ixP) * a.iyrmax[p] * (own + gt);
            }
            if (U > 0.f) sc = ldexpf(1.0f, max(-126, min(126, 14 - (ilogbf(U) + 1))));
        }
        const float rsig = 1.0f / a.oSig[orow];  // exact: sig is a power of two
#pragma unroll
        for (int p = 0; p < NPV; ++p) {
            const int pp = p < P ? p : 0;
            Ao[p] = a.oA[pp * a.NO + orow] * rsig;
            const float c = a.oC[pp * a.NO + orow];
            Co[p] = SIG ? c * sc : c + log2f(sc);
            Ro[p] = SIG ? 0.f : a.oRho[pp * a.NO + orow];
        }
        csc = rsig / sc;
        if (w == 0 && h == 0) inv_sc[l32] = 1.0f / sc;
    }

    // ---- copies of inner block nb into ring slot sl: this wave's rows 4 w .. 4 w + 3 (the FP16
    // inner matrix carries two zero blocks past its last row), their first DC columns (the steps
    // of the four waves; later columns are never read) in 1 KB pieces, and one float of the
    // block's tables [iI | iKap][p][row] per lane (rows past the end read the last row)
    const int DC = min(D, 4 * NQ * 32);
    const int npc = (DC * 2 + 1023) / 1024;
    const int lastc = (DC * 2 - (npc - 1) * 1024) / 16;  // active lanes of the last piece
    const uint32_t ys_lds = (uint32_t)(uintptr_t)&Ys[0][0];
    const int te = 64 * w + lane;
    const bool tact = te < 2 * P * BI;
    const int tr = te % BI;
    const float *tbase = tact ? ((te / (P * BI)) == 0 ? a.iI : a.iKap) + (int64_t)((te / BI) % P) * NI + tr : a.iI;
    const int tlim = tact ? NI - 1 - tr : 0;
    auto issue_block = [&](int nb, int sl) {
        const _Float16 *gblk = a.Y16 + (int64_t)nb * BI * D;
        for (int k = 0; k < 4; ++k) {
            // swizzled: lane i of a 1 KB piece fetches the chunk that belongs at chunk i (every piece full)
            const int src_lane = SWZ ? (lane ^ gen_swz(4 * w + k)) : lane;
            const uint32_t voff = (uint32_t)(4 * w + k) * (uint32_t)D * 2u + 16u * (uint32_t)src_lane;
            const uint32_t m0v = __builtin_amdgcn_readfirstlane(ys_lds + 2u * (uint32_t)(sl * RSL + (4 * w + k) * YP));
            for (int pc = 0; pc < npc; ++pc)
                if (pc + 1 < npc || lane < lastc) dma_row1(gblk, voff + 1024u * pc, m0v + 1024u * pc);
        }
        const uint32_t tb = __builtin_amdgcn_readfirstlane(ys_lds + 2u * (uint32_t)(sl * RSL + BI * YP) + 4u * (uint32_t)(64 * w));
        dma4_m0(tbase + min(nb * BI, tlim), tb);
    };

    // zero the ring (tile columns past D stay zero) and the bands (band P stays zero)
    for (int e = tid; e < 2 * RSL / 8; e += 256) *(uint4 *)&Ys[0][e * 8] = make_uint4(0, 0, 0, 0);
    for (int e = tid; e < G::NBAND * GBO * APITCH / 8; e += 256) *(uint4 *)&At[0][e * 8] = make_uint4(0, 0, 0, 0);
    lds_barrier();

    // ---- outer rows' columns of this wave's steps as B operands (zero past NO or D)
    f16x8 xr[2][NQ];
#pragma unroll
    for (int ob = 0; ob < 2; ++ob) {
        const int orow = o0 + 16 * ob + l16;
#pragma unroll
        for (int ks = 0; ks < NQ; ++ks) {
            const int d = dq0 + 32 * ks + 8 * g4;
            f16x8 v = {};
            if (orow < NO && d < D) v = *(const f16x8 *)(a.X16 + (int64_t)orow * D + d);
            xr[ob][ks] = v;
        }
    }
    f32x16 dacc[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) dacc[j][r] = 0.f;
    float Cacc[NPV], Lacc[NPV], Bacc[NPV];
#pragma unroll
    for (int p = 0; p < NPV; ++p) Cacc[p] = Lacc[p] = Bacc[p] = 0.f;

    // listed cells: the entries of this workgroup's 64-row table block, sorted by nb
    const int lob = (int)blockIdx.x >> 1, lbit = 32 * ((int)blockIdx.x & 1) + l32;
    int lcur = 0, lend = 0;
    if (a.lptr) {
        lcur = a.lptr[lob];
        lend = a.lptr[lob + 1];
    }
    int lnb = lcur < lend ? a.lent[lcur].nb : INT_MAX;
    auto listed = [&](int nb) {
        while (lnb < nb) {
            ++lcur;
            lnb = lcur < lend ? a.lent[lcur].nb : INT_MAX;
        }
        return lnb == nb;
    };

    // transposed reads of the inner tile for the update (per-lane part; slot and step added)
    const _Float16 *ytr = &Ys[0][0] + (8 * (g4 >> 1) + (l16 >> 2)) * YP + 16 * (g4 & 1) + 4 * (lane & 3) + dq0;
    const float *tabs0 = (const float *)&Ys[0][BI * YP];

    uint64_t wbands = 0;  // the compiled ladder's bands of this wave's steps
    if constexpr (LM != 0) {
        using GL = GenLadder<LM, NQ>;
        constexpr uint64_t b0 = GL::bands(0), b1 = GL::bands(1), b2 = GL::bands(2), b3 = GL::bands(3);
        wbands = w == 0 ? b0 : w == 1 ? b1 : w == 2 ? b2 : b3;
        wbands = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(wbands >> 32)) << 32) |
                 (uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)wbands);
    }

    if (nb_begin < nb_end) {
        issue_block(nb_begin, 0);
        wait_vm();
        lds_barrier();
    }
    for (int nb = nb_begin; nb < nb_end; ++nb) {
        const int cur = (nb - nb_begin) & 1;
        issue_block(nb + 1, cur ^ 1);  // past the end: a zero block or the next split's rows, unused

        // recompute: partial S^T (16 inner x 32 outer) over this wave's steps, and a snapshot
        // after each step where a prefix ends inside them
        {
            const _Float16 *yrow = &Ys[cur][0] + l16 * YP + dq0 + 8 * g4;
            f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
            auto put = [&](int slot) {
#pragma unroll
                for (int ob = 0; ob < 2; ++ob) *(f32x4 *)&Sl[slot][(16 * ob + l16) * SLOTP + 4 * g4] = acc[ob];
            };
            if constexpr (LM != 0) {
                // the ladder's snapshots are known per step: straight-line steps with the tile
                // reads RD steps ahead
                using GL = GenLadder<LM, NQ>;
                constexpr int RD = NQ < 4 ? NQ : (SIG ? 2 : 4);  // the sigmoid form has fewer registers to spare
                // step ks reads logical chunk 4 ks + g4 of row l16, stored at 4 (ks ^ (sw >> 2)) + (g4 ^ (sw & 3))
                const int sw = gen_swz(l16);
                const _Float16 *yr0 = &Ys[cur][0] + l16 * YP + dq0 + 8 * (g4 ^ (sw & 3));
                const _Float16 *yrm[4] = {yr0 + 32 * (0 ^ (sw >> 2)), yr0 + 32 * (1 ^ (sw >> 2)), yr0 + 32 * (2 ^ (sw >> 2)),
                                          yr0 + 32 * (3 ^ (sw >> 2))};
                auto yat = [&](int ks) { return (const f16x8 *)(yrm[ks & 3] + 32 * (ks & ~3)); };
                f16x8 yb[RD];
                static_for<0, RD>([&](auto kc) { yb[decltype(kc)::value] = *yat(decltype(kc)::value); });
                static_for<0, NQ>([&](auto kc) {
                    constexpr int ks = decltype(kc)::value;
                    const f16x8 yv = yb[ks % RD];
                    if constexpr (ks + RD < NQ) yb[ks % RD] = *yat(ks + RD);
#pragma unroll
                    for (int ob = 0; ob < 2; ++ob)
                        acc[ob] = __builtin_amdgcn_mfma_f32_16x16x32_f16(yv, xr[ob][ks], acc[ob], 0, 0, 0);
                    constexpr uint32_t wm = GL::snap_waves(ks);
                    if constexpr (wm != 0u) {
                        static_for<0, 4>([&](auto Wc) {
                            constexpr int W = decltype(Wc)::value;
                            constexpr int slot = GL::snap_at(W * NQ + ks);
                            if constexpr (slot >= 0)
                                if (w == W) put(slot);
                        });
                    }
                });
            } else {
#pragma unroll
                for (int ks = 0; ks < NQ; ++ks) {
                    const f16x8 yv = *(const f16x8 *)(yrow + 32 * ks);
#pragma unroll
                    for (int ob = 0; ob < 2; ++ob)
                        acc[ob] = __builtin_amdgcn_mfma_f32_16x16x32_f16(yv, xr[ob][ks], acc[ob], 0, 0, 0);
                    const int sl = a.gt.snap_at[w * NQ + ks];
                    if (sl >= 0) put(sl);
                }
            }
            put(w);
        }
        lds_barrier();

        // epilogue: coefficients of this lane's two cells for every prefix, widest first
        {
            const int nl = 4 * w + 2 * h;  // row of the first cell in the block
            const float *tab = (const float *)((const char *)tabs0 + cur * RSL * 2);
            bool ok[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int n = nb * BI + nl + t;
                ok[t] = ovalid && n < NI && n != ((o + dsh) ^ pxr) && (pxr == 0 || n != o + dsh);
            }
            if (listed(nb)) {
                const uint64_t *lm = a.lent[lcur].m + nl;
#pragma unroll
                for (int t = 0; t < 2; ++t) ok[t] = ok[t] && ((lm[t] >> lbit) & 1ull) == 0ull;
            }
            float run[2] = {0.f, 0.f};
            // the unit of prefix p (a compile-time index, so that the per-prefix registers stay
            // registers), given S^p: the full partials of the waves below the one where p ends, plus
            // p's snapshot slot
            auto unit = [&](auto pc, f32x2 Sp) {
                constexpr int p = decltype(pc)::value;
                float av[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const float iy = tab[p * BI + nl + t];
                    const float e = Sp[t] * Ao[p];
                    float c;
                    if constexpr (!SIG) {
                        c = __builtin_amdgcn_exp2f(fmaf(e, iy, Co[p])) * fmaf(Ro[p], iy, tab[(P + p) * BI + nl + t]);
                    } else {
                        const float uu = fmaf(e, iy, a.b2);
                        const float tt = __builtin_amdgcn_exp2f(-fabsf(uu));
                        const float wq = 1.f + tt;
                        const float rr = __builtin_amdgcn_rcpf(wq);
                        const float sg = uu >= 0.f ? rr : tt * rr;
                        c = sg * Co[p] * iy;  // Co holds beta_o for the sigmoid form
                        if (want_loss && ok[t]) {
                            // softplus(l) / ln 2 = max(u, 0) + log2(1 + tt), with log1p's rounding corrected
                            Lacc[p] += fmaxf(uu, 0.f) + __builtin_amdgcn_logf(wq) + (tt - (wq - 1.f)) * rr * kLog2e;
                            if (want_bias) Bacc[p] += sg;
                        }
                    }
                    av[t] = ok[t] ? c : 0.f;
                    run[t] += av[t];
                    Cacc[p] = fmaf(av[t], Sp[t], Cacc[p]);
                }
                uint32_t hpk;
                asm("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(hpk) : "v"(run[0]), "v"(run[1]));
                *(uint32_t *)&At[p][l32 * APITCH + nl] = hpk;
            };
            if constexpr (LM != 0) {  // the ladder known at compile time: fixed slots, no loops
                using GL = GenLadder<LM, NQ>;
                static_for<0, GL::P>([&](auto ic) {
                    constexpr int p = GL::P - 1 - decltype(ic)::value;
                    constexpr int slot = GL::snap_slot(p), wv = GL::wave_of(p);
                    f32x2 Sp = *(const f32x2 *)&Sl[slot][l32 * SLOTP + nl];
                    static_for<0, wv>(
                        [&](auto qc) { Sp += *(const f32x2 *)&Sl[decltype(qc)::value][l32 * SLOTP + nl]; });
                    unit(std::integral_constant<int, p>{}, Sp);
                });
            } else {
                static_for<0, kMaxP>([&](auto ic) {
                    constexpr int p = kMaxP - 1 - decltype(ic)::value;
                    if (p >= P) return;
                    const int wv = a.gt.wave_of[p];
                    f32x2 Sp = *(const f32x2 *)&Sl[a.gt.snap_slot[p]][l32 * SLOTP + nl];
                    for (int q = 0; q < wv; ++q) Sp += *(const f32x2 *)&Sl[q][l32 * SLOTP + nl];
                    unit(std::integral_constant<int, p>{}, Sp);
                });
            }
        }
        lds_barrier();

        // update: dX[:, this wave's steps] += A_band . Y
        if constexpr (UPD && LM != 0) {
            // the bands of every wave's steps are known (4 bits per step, this wave's sequence in
            // scalar registers); the band and tile reads run RD steps ahead of the products
            using GL = GenLadder<LM, NQ>;
            constexpr int RD = NQ < 3 ? NQ : (SIG ? 2 : 3);
            // row ru = 8 (g4 >> 1) + (l16 >> 2) (and ru + 4, whose swizzle is sw ^ 8) at logical
            // chunk 4 jb + t, t = 2 (g4 & 1) + ((lane & 3) >> 1), half lane & 1 of it
            const int ru = 8 * (g4 >> 1) + (l16 >> 2), sw = gen_swz(ru);
            const _Float16 *yu0 = &Ys[cur][0] + ru * YP + dq0 + 8 * ((2 * (g4 & 1) + ((lane & 3) >> 1)) ^ (sw & 3)) +
                                  4 * (lane & 1);
            const _Float16 *yum[4] = {yu0 + 32 * (0 ^ (sw >> 2)), yu0 + 32 * (1 ^ (sw >> 2)), yu0 + 32 * (2 ^ (sw >> 2)),
                                      yu0 + 32 * (3 ^ (sw >> 2))};
            const _Float16 *asrc = &At[0][0] + l32 * APITCH + 8 * h;
            f16x8 ab[RD];
            f16x4 ylo[RD], yhi[RD];
            auto rd = [&](auto jc) {
                constexpr int jb = decltype(jc)::value;
                const int band = (int)((wbands >> (4 * jb)) & 15u);
                ab[jb % RD] = *(const f16x8 *)(asrc + band * (GBO * APITCH));
                ylo[jb % RD] = ds_read_tr(yum[jb & 3] + 32 * (jb & ~3));
                yhi[jb % RD] = ds_read_tr(yum[(jb & 3) ^ 2] + 32 * (jb & ~3) + 4 * YP);
            };
            static_for<0, RD>(rd);
            static_for<0, NQ>([&](auto jc) {
                constexpr int jb = decltype(jc)::value;
                const f16x8 af = ab[jb % RD];
                const f16x8 bfv = __builtin_shufflevector(ylo[jb % RD], yhi[jb % RD], 0, 1, 2, 3, 4, 5, 6, 7);
                if constexpr (jb + RD < NQ) rd(std::integral_constant<int, jb + RD>{});
                dacc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bfv, dacc[jb], 0, 0, 0);
            });
        } else if constexpr (UPD) {
#pragma unroll
            for (int jb = 0; jb < NQ; ++jb) {
                const int band = a.gt.band_of[w * NQ + jb];
                const f16x8 af = *(const f16x8 *)&At[band][l32 * APITCH + 8 * h];
                const _Float16 *ysrc = ytr + cur * RSL + 32 * jb;
                const f16x4 lo = ds_read_tr(ysrc);
                const f16x4 hi = ds_read_tr(ysrc + 4 * YP);
                const f16x8 bfv = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                dacc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bfv, dacc[jb], 0, 0, 0);
            }
        }
        wait_vm();      // the copies of block nb + 1 landed
        lds_barrier();  // ... for every wave; the slots and bands of block nb are consumed
    }

    // ---- the raw gradient block (scale divided out) into this split's partial
    const int64_t split = blockIdx.y;
    if constexpr (UPD) {
        float *dst = a.part + split * a.NO * D;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int orow = 8 * (r >> 2) + 4 * h + (r & 3);
            const float sv = inv_sc[orow];
            if (o0 + orow < NO) {
                float *rowp = dst + (int64_t)(o0 + orow) * D + dq0 + l32;
#pragma unroll
                for (int jb = 0; jb < NQ; ++jb)
                    if (dq0 + 32 * jb + l32 < D) rowp[32 * jb] = dacc[jb][r] * sv;
            }
        }
    }
    // radial sums over the eight (wave, half) parts of each row, and the sigmoid loss sums
    float *red = &Sl[0][0];  // [8][kMaxP][GBO], then [4][kMaxP] twice
#pragma unroll
    for (int p = 0; p < NPV; ++p) red[((2 * w + h) * kMaxP + p) * GBO + l32] = Cacc[p];
    if (want_loss) {
#pragma unroll
        for (int p = 0; p < NPV; ++p) {
            const float v = wave_sum(Lacc[p]), u = wave_sum(Bacc[p]);
            if (lane == 0) {
                red[8 * kMaxP * GBO + w * kMaxP + p] = v;
                red[8 * kMaxP * GBO + 4 * kMaxP + w * kMaxP + p] = u;
            }
        }
    }
    lds_barrier();
    if (w == 0 && h == 0 && ovalid) {
        for (int p = 0; p < P; ++p) {
            float c = 0.f;
            for (int k = 0; k < 8; ++k) c += red[(k * kMaxP + p) * GBO + l32];
            a.Cpart[(split * P + p) * a.NO + o] = c * csc;
        }
    }
    if (want_loss && tid < P) {
        const float *lr = red + 8 * kMaxP * GBO;
        const int64_t slot = (int64_t)a.loss_slot0 + split * gridDim.x + blockIdx.x;
        a.lossparts[slot * P + tid] =
            (((lr[0 * kMaxP + tid] + lr[1 * kMaxP + tid]) + lr[2 * kMaxP + tid]) + lr[3 * kMaxP + tid]) * kLn2;
        if (want_bias) {
            const float *br = lr + 4 * kMaxP;
            a.biasparts[slot * P + tid] =
                ((br[0 * kMaxP + tid] + br[1 * kMaxP + tid]) + br[2 * kMaxP + tid]) + br[3 * kMaxP + tid];
        }
    }
}

// ----------------------------------------------------------------------------
// k_maxes: gmax[t][p] = max over the rows of table t, prefix p (one block each;
// a fixed tree, so the result does not depend on scheduling).
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_maxes(const float *t0, const float *t1, const float *t2, const float *t3,
                                               int64_t n0, int64_t n1, int64_t n2, int64_t n3, int P, int chunks,
                                               float *gmax) {
    // block (t, p, c) takes chunk c of table t, prefix p; gmax starts at 0 (k_prep) and takes
    // each chunk's maximum by an integer maximum of the bit patterns (the values are >= 0, so
    // the order of the bits is the order of the values, and the result does not depend on
    // the order of the blocks)
    __shared__ float red[256];
    const int c = blockIdx.x % chunks, tp = blockIdx.x / chunks;
    const int t = tp / P, p = tp % P;
    const float *src = t == 0 ? t0 : t == 1 ? t1 : t == 2 ? t2 : t3;
    const int64_t n = t == 0 ? n0 : t == 1 ? n1 : t == 2 ? n2 : n3;
    const int64_t per = (n + chunks - 1) / chunks, b = c * per, e = b + per < n ? b + per : n;
    float m = 0.f;
    if (src)
        for (int64_t i = b + threadIdx.x; i < e; i += 256) m = fmaxf(m, src[p * n + i]);
    red[threadIdx.x] = m;
    __syncthreads();
    for (int h = 128; h >= 1; h >>= 1) {
        if ((int)threadIdx.x < h) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + h]);
        __syncthreads();
    }
    if (threadIdx.x == 0) atomicMax((int *)&gmax[t * P + p], __float_as_int(red[0]));
}

// ----------------------------------------------------------------------------
// k_finalize: per outer row, sum the split partials and add the exact FP32
// terms: the positive cell (left out of the band operands) and the radial
// part of the normalisation Jacobian, -x[d] sum_{p: P_p > d} ix_p^2 C^p.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_finalize(FinArgs a) {
    __shared__ float DG[kMaxP], RD[kMaxP];
    __shared__ float Cs[kMaxP];
    const int64_t o = blockIdx.x;
    const int P = a.pf.n;
    const int D = a.D;
    const int Dw = a.pf.w[P - 1];
    const int64_t ipos = o + a.pos_shift;  // index of the positive's query row in diagA/posdot
    const bool has_pos = ipos >= 0 && ipos < a.R;
    const int64_t ypos = (o + a.diag_shift) ^ a.pxor;  // positive's row in Y
    // This thread's columns: groups of four, 4 (tid + 256 g) (prefix ends are multiples of 32,
    // so a group lies in one band).  Their split partials and row values are loaded first, so
    // that those loads are in flight during the table work below.
    constexpr int GMAX = kMaxD / 1024;
    float4 pv[GMAX];
    uint2 xw[GMAX], yw[GMAX];
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
        const int d0 = 4 * ((int)threadIdx.x + 256 * g);
        pv[g] = make_float4(0.f, 0.f, 0.f, 0.f);
        xw[g] = yw[g] = make_uint2(0u, 0u);
        if (d0 < Dw) {
            for (int64_t sp = 0; sp < a.nsplit; ++sp) {
                const float4 u = *(const float4 *)(a.part + (sp * a.NO + o) * D + d0);
                pv[g].x += u.x;
                pv[g].y += u.y;
                pv[g].z += u.z;
                pv[g].w += u.w;
            }
            xw[g] = *(const uint2 *)(a.X + o * D + d0);
            if (has_pos) yw[g] = *(const uint2 *)(a.Y + ypos * D + d0);
        }
    }
    // radial sums over the splits: wave p adds prefix p's partials (a fixed order per lane,
    // then a fixed tree across the lanes)
    {
        const int wv = threadIdx.x >> 6, ln = threadIdx.x & 63;
        for (int p = wv; p < P; p += 4) {
            float c = 0.f;
            for (int64_t sp = ln; sp < a.nsplit; sp += 64) c += a.Cpart[(sp * P + p) * a.NO + o];
            c = wave_sum(c);
            if (ln == 0) Cs[p] = c;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float dg = 0.f, rd = 0.f, ts = 0.f;
        for (int p = P - 1; p >= 0; --p) {
            const float C = Cs[p];
            float dA = 0.f, dS = 0.f;
            if (has_pos) {
                dA = a.diagA[p * a.R + ipos];
                dS = a.posdot[p * a.R + ipos];
            }
            const float ix = a.invx[p * a.NO + o];
            // radial coefficient of prefix p: (w_p / W) s sum_j g_oj cos_oj, the positive cell included
            const float T = fmaf(dA, dS, C * a.gam[o]);
            dg += dA;
            rd += ix * ix * T;
            ts += T;
            DG[p] = dg;
            RD[p] = rd;
        }
        if (a.tsum) a.tsum[o] = ts;
    }
    __syncthreads();
    const float gm = a.gam[o];
    float *dst = a.out + o * D;
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
        const int d0 = 4 * ((int)threadIdx.x + 256 * g);
        if (d0 >= D) break;
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        if (d0 < Dw) {
            int b = 0;
            while (d0 >= a.pf.w[b]) ++b;
            const float dgb = DG[b], rdb = RD[b];
            const float p4[4] = {pv[g].x, pv[g].y, pv[g].z, pv[g].w};
            const unsigned int xu[2] = {xw[g].x, xw[g].y}, yu[2] = {yw[g].x, yw[g].y};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float xv = (e & 1) ? bf16_hi(xu[e >> 1]) : bf16_lo(xu[e >> 1]);
                const float yv = (e & 1) ? bf16_hi(yu[e >> 1]) : bf16_lo(yu[e >> 1]);
                v[e] = fmaf(dgb, yv, fmaf(-rdb, xv, p4[e] * gm));
            }
        }
        float4 *dp = (float4 *)(dst + d0);
        if (a.accumulate) {
            const float4 old = *dp;
            v[0] += old.x;
            v[1] += old.y;
            v[2] += old.z;
            v[3] += old.w;
        }
        *dp = make_float4(v[0], v[1], v[2], v[3]);
    }
}

// ----------------------------------------------------------------------------
// k_loss: fixed-order sum of every loss partial slot -> loss and L^p.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_loss(LossArgs a) {
    __shared__ double red[256];
    __shared__ double lp[kMaxP];
    const int P = a.pf.n;
    for (int p = 0; p < P; ++p) {
        double v = 0.0;
        for (int64_t s = threadIdx.x; s < a.nslots; s += 256) v += (double)a.lossparts[s * P + p];
        red[threadIdx.x] = v;
        __syncthreads();
        for (int h = 128; h >= 1; h >>= 1) {
            if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
            __syncthreads();
        }
        if (threadIdx.x == 0) lp[p] = red[0] * a.norm;
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        double tot = 0.0;
        for (int p = 0; p < P; ++p) {
            tot += (double)a.wnorm[p] * lp[p];
            if (a.prefix_losses_out) a.prefix_losses_out[p] = (float)lp[p];
        }
        *a.loss_out = (float)tot;
    }
    // dL/dscale = (1/s) sum over the rows of one backward pass of sum_p (w_p / W) s sum_j g cos
    if (a.dscale_out) {
        double v = 0.0;
        for (int64_t o = threadIdx.x; o < a.ntsum; o += 256) v += (double)a.tsum[o];
        __syncthreads();
        red[threadIdx.x] = v;
        __syncthreads();
        for (int h = 128; h >= 1; h >>= 1) {
            if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
            __syncthreads();
        }
        if (threadIdx.x == 0) *a.dscale_out = (float)(red[0] * (double)a.inv_scale);
        __syncthreads();
    }
    // dL/dbias = sum_p (w_p / W) sum_ij g_ij: zero for a softmax (a common shift of a row's or a
    // column's logits cancels); for the sigmoid form (sum of sigma(l) - number of positives) / N
    if (a.dbias_out) {
        double tot = 0.0;
        for (int p = 0; p < P && a.biasparts; ++p) {
            double v = 0.0;
            for (int64_t s = threadIdx.x; s < a.nslots; s += 256) v += (double)a.biasparts[s * P + p];
            __syncthreads();
            red[threadIdx.x] = v;
            __syncthreads();
            for (int h = 128; h >= 1; h >>= 1) {
                if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
                __syncthreads();
            }
            tot += (double)a.wnorm[p] * red[0] * a.norm;
            __syncthreads();
        }
        if (threadIdx.x == 0) *a.dbias_out = (float)tot;
    }
}

// ----------------------------------------------------------------------------
// launch wrappers (host side of this translation unit)
// ----------------------------------------------------------------------------
hipError_t launch_prep(const PrepArgs &a, hipStream_t s) {
    const int64_t rows = a.R + a.N;
    // 16 rows per wave where that still gives 1024 workgroups, else 4, else 1; rows wider than
    // 1024 take four chunk groups per lane
    const bool wide = a.D > 1024;
    if (rows >= 1024 * kPrepRows) {
        if (wide) hipLaunchKernelGGL((k_prep<16, 4>), dim3((unsigned)((rows + 63) / 64)), dim3(256), 0, s, a);
        else hipLaunchKernelGGL((k_prep<16, 2>), dim3((unsigned)((rows + 63) / 64)), dim3(256), 0, s, a);
    } else if (rows >= 1024 * 16) {
        if (wide) hipLaunchKernelGGL((k_prep<4, 4>), dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, s, a);
        else hipLaunchKernelGGL((k_prep<4, 2>), dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, s, a);
    } else {
        if (wide) hipLaunchKernelGGL((k_prep<1, 4>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a);
        else hipLaunchKernelGGL((k_prep<1, 2>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

// Prefix ladders with a compiled backward (bit ds set: a prefix ends at 32 (ds + 1)).
#define UFORM_LADDERS(X)                                                        \
    X(0x8000808Au) /* 64, 128, 256, 512, 1024 */                                \
    X(0x0000808Au) /* 64, 128, 256, 512 */                                      \
    X(0x0000008Au) /* 64, 128, 256 */                                           \
    X(0x0000000Au) /* 64, 128 */                                                \
    X(0x80000000u) /* 1024 */                                                   \
    X(0x00008000u) /* 512 */                                                    \
    X(0x00000080u) /* 256 */                                                    \
    X(0x00000008u) /* 128 */

hipError_t launch_fwd(const u16 *q, const u16 *k, int64_t R, int64_t N, int D, const Prefixes &pf, int64_t off,
                      const float *rowA, const float *colI, float cshift, float *rowpart, float *colpart,
                      float *posdot, hipStream_t s) {
    const int64_t nIt = (R + FB - 1) / FB, nJt = (N + FB - 1) / FB;
    uint64_t mask = 0;  // bit e: a prefix ends at 32 (e + 1) (widths up to 2048)
    for (int p = 0; p < pf.n; ++p) mask |= 1ull << (pf.w[p] / 32 - 1);
    const dim3 grid((unsigned)(nIt * nJt));
    if (mask == kLadder2048) {  // the Large and XL tiers' ladder
        hipLaunchKernelGGL(k_fwd<fwd_ladder(kLadder2048)>, grid, dim3(256), 0, s, q, k, R, N, D, pf, off, rowA, colI,
                           cshift, rowpart, colpart, posdot);
        return hipGetLastError();
    }
#define UFORM_CASE(m)                                                                                          \
    if (fwd_ladder(m) != 0ull && mask == (m)) {                                                                \
        hipLaunchKernelGGL(k_fwd<fwd_ladder(m)>, grid, dim3(256), 0, s, q, k, R, N, D, pf, off, rowA, colI, cshift, \
                           rowpart, colpart, posdot);                                                          \
        return hipGetLastError();                                                                              \
    }
    UFORM_LADDERS(UFORM_CASE)
#undef UFORM_CASE
    hipLaunchKernelGGL(k_fwd<0ull>, grid, dim3(256), 0, s, q, k, R, N, D, pf, off, rowA, colI, cshift, rowpart,
                       colpart, posdot);
    return hipGetLastError();
}

hipError_t launch_rowstats(const StatsArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(k_rowstats, dim3((unsigned)((a.R + kStatRows - 1) / kStatRows)), dim3(64 * stat_waves(a.nJt)), 0,
                       s, a);
    return hipGetLastError();
}

hipError_t launch_colstats(const StatsArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(k_colstats, dim3((unsigned)((a.N + kStatRows - 1) / kStatRows)), dim3(64 * stat_waves(a.nIt)), 0,
                       s, a);
    return hipGetLastError();
}

hipError_t launch_siglip_tabs(const StatsArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(k_siglip_tabs, dim3((unsigned)((a.R + a.N + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <uint32_t MASK, bool LIST>
static hipError_t launch_bwd_sig(const BwdArgs &a, dim3 grid, hipStream_t s) {
    const bool bias = a.biasparts != nullptr;
    if (a.do_update && a.want_loss && bias)
        hipLaunchKernelGGL((k_bwd<MASK, true, true, true, true, LIST>), grid, dim3(256), 0, s, a);
    else if (a.do_update && a.want_loss)
        hipLaunchKernelGGL((k_bwd<MASK, true, true, true, false, LIST>), grid, dim3(256), 0, s, a);
    else if (a.do_update)
        hipLaunchKernelGGL((k_bwd<MASK, true, true, false, false, LIST>), grid, dim3(256), 0, s, a);
    else if (bias)
        hipLaunchKernelGGL((k_bwd<MASK, true, false, true, true, LIST>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((k_bwd<MASK, true, false, true, false, LIST>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

template <uint32_t MASK>
static hipError_t launch_bwd_mask(const BwdArgs &a, bool sig, dim3 grid, hipStream_t s) {
    if (!sig) {
        hipLaunchKernelGGL((k_bwd<MASK, false, true, false, false, false>), grid, dim3(256), 0, s, a);
        return hipGetLastError();
    }
    return a.lptr ? launch_bwd_sig<MASK, true>(a, grid, s) : launch_bwd_sig<MASK, false>(a, grid, s);
}

bool bwd_mask_supported(uint32_t mask) {
#define UFORM_CASE(m) if (mask == (m)) return true;
    UFORM_LADDERS(UFORM_CASE)
#undef UFORM_CASE
    return false;
}

hipError_t launch_bwd(const BwdArgs &a, uint32_t mask, bool sig, int64_t nsplit, hipStream_t s) {
    const dim3 grid((unsigned)((a.NO + BO - 1) / BO), (unsigned)nsplit);
#define UFORM_CASE(m) \
    if (mask == (m)) return launch_bwd_mask<(m)>(a, sig, grid, s);
    UFORM_LADDERS(UFORM_CASE)
#undef UFORM_CASE
    return hipErrorInvalidValue;
}

template <int NQ>
static hipError_t launch_bwd_gen_nq(const BwdArgs &a, bool sig, dim3 grid, hipStream_t s) {
    uint64_t lm = 0;  // the ladder as a 64-bit mask (prefix ends at multiples of 32 up to 2048)
    for (int p = 0; p < a.pf.n; ++p) lm |= 1ull << (a.pf.w[p] / 32 - 1);
    if constexpr (NQ == 16) {
        if (lm == kLadder2048 && a.D == 2048) {  // compiled with the ladder's slots and a swizzled ring
            if (!sig)
                hipLaunchKernelGGL((k_bwd_gen<NQ, false, true, kLadder2048>), grid, dim3(256), 0, s, a);
            else if (a.do_update)
                hipLaunchKernelGGL((k_bwd_gen<NQ, true, true, kLadder2048>), grid, dim3(256), 0, s, a);
            else
                hipLaunchKernelGGL((k_bwd_gen<NQ, true, false, kLadder2048>), grid, dim3(256), 0, s, a);
            return hipGetLastError();
        }
    }
    if (!sig)
        hipLaunchKernelGGL((k_bwd_gen<NQ, false, true>), grid, dim3(256), 0, s, a);
    else if (a.do_update)
        hipLaunchKernelGGL((k_bwd_gen<NQ, true, true>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((k_bwd_gen<NQ, true, false>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_bwd_gen(const BwdArgs &a, int nq, bool sig, int64_t nsplit, hipStream_t s) {
    const dim3 grid((unsigned)((a.NO + GBO - 1) / GBO), (unsigned)nsplit);
    switch (nq) {
        case 1: return launch_bwd_gen_nq<1>(a, sig, grid, s);
        case 2: return launch_bwd_gen_nq<2>(a, sig, grid, s);
        case 4: return launch_bwd_gen_nq<4>(a, sig, grid, s);
        case 8: return launch_bwd_gen_nq<8>(a, sig, grid, s);
        case 16: return launch_bwd_gen_nq<16>(a, sig, grid, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_maxes(const float *t0, const float *t1, const float *t2, const float *t3, int64_t n0, int64_t n1,
                        int64_t n2, int64_t n3, int P, float *gmax, hipStream_t s) {
    int64_t nmax = n0 > n1 ? n0 : n1;
    nmax = nmax > n2 ? nmax : n2;
    nmax = nmax > n3 ? nmax : n3;
    const int chunks = (int)(nmax / 4096 < 1 ? 1 : (nmax / 4096 > 64 ? 64 : nmax / 4096));
    hipLaunchKernelGGL(k_maxes, dim3((unsigned)(4 * P * chunks)), dim3(256), 0, s, t0, t1, t2, t3, n0, n1, n2, n3, P,
                       chunks, gmax);
    return hipGetLastError();
}

hipError_t launch_finalize(const FinArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(k_finalize, dim3((unsigned)a.NO), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_loss(const LossArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(k_loss, dim3(1), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace uform
