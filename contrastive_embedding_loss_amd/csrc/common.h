// Types and kernel argument blocks shared by the kernels and the host library.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace uform {

using u16 = unsigned short;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kMaxP = 8;
constexpr int kMaxD = 2048;
constexpr int kMaxSteps = kMaxD / 32;  // 32-wide steps of the widest row
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

constexpr int kInfonce = 0;
constexpr int kSiglip = 1;
constexpr int kRows = 2;
constexpr int kOneset = 3;  // one-set sigmoid form: computed as the sigmoid kind with pxor = 1, mirror = 2
constexpr int kOnesetEdges = 4;  // one-set form with listed relations only: pxor = 0, mirror = 2, no implicit positive

__host__ __device__ inline bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

struct Prefixes {
    int n;
    int w[kMaxP];
};

// k_prep outputs.  sig = 2^-floor(log2 |row[:P_last]|) (exact power of two),
// gam = |s| inv_P / den (per-row scale of the backward's band operand),
// iyr = inv_p / sig.
struct PrepArgs {
    const u16 *q, *k;
    int64_t R, N, off;
    int pxor;  // positive of local row i: key (off + i) ^ pxor (1: the one-set form's pairs)
    int want_pos;  // 1: the positive dot products (posdot) are formed here; 0: the forward writes them
    int D;
    Prefixes pf;
    float a_scale, gam_scale;
    float *invq, *invk, *qA, *kA, *qIYR, *kIYR, *posdot, *sigq, *sigk, *gamq, *gamk;
    float *gmax;  // [4][P], zeroed here for k_maxes
    // sig-scaled FP16 copies of the rows for the backward (nullptr: no backward runs), with their
    // zero rows up to Rpad and Npad (the backward's copies run past the last block)
    _Float16 *qH, *kH;
    int64_t Rpad, Npad;
};

// Statistics / coefficient-table kernels.  "q" tables are [P][R], "k" tables [P][N].
struct StatsArgs {
    int64_t R, N, off, nJt, nIt;
    int pxor;      // as in PrepArgs
    int nopos;     // 1: no implicit positive (one-set form with listed relations): no positive-cell terms
    float mirror;  // 2 for the one-set form (a row's gradient through both mirrored cells), else 1
    Prefixes pf;
    int kind;
    float scale, bias, cshift, lse_offset, inv_den, sgn;
    float wnorm[kMaxP];  // w_p / W
    const float *rowpart, *colpart;
    const float *invq, *invk, *posdot, *qA;
    float *row_lse_out, *col_lse_out, *pos_logit_out;
    float *negfrac;           // [P][R]: (1 - p_ii) of the row softmax
    float *kNegfrac;          // [P][N]: negative mass fraction of each column's softmax
    const float *qIYR, *kIYR;
    float *qC, *qRho, *qKap;  // query-side tables
    float *kC, *kRho, *kKap;  // key-side tables
    float *diagA;             // [P][R]: exact coefficient of the positive cell
    float *lossparts;         // [slot][P]
    float *biasparts;         // sigmoid form: [slot][P], minus the positives' sigma(-l); nullable
    int64_t slot0;
};

// Listed cells (extra positives) of one (outer block of 64 rows, inner block of 16 rows) pair of a
// backward pass: bit o of m[r] marks the cell of outer row 64 ob + o and inner row 16 nb + r.  A
// pass's entries are sorted by outer block, then by nb (one entry per pair); the backward leaves
// these cells out of its band operands and sums, and the extra-positive pass gives them their whole
// loss and residual in FP32.
struct ListEnt {
    int32_t nb, pad;
    uint64_t m[16];
};
constexpr int kListEntWords = (int)(sizeof(ListEnt) / 4);
static_assert(sizeof(ListEnt) == 136, "ListEnt layout");

// Tables of the generic backward (any prefix ladder): wave w of its workgroup owns the 32-wide
// steps [w nq, (w + 1) nq) of the widest prefix.  S^p = the full partials of the waves below
// wave_of[p] plus slot snap_slot[p] (wave_of[p]'s full partial when prefix p ends on its last
// step, else a snapshot taken after step snap_at == snap_slot).
struct GenTabs {
    int8_t wave_of[kMaxP];
    int8_t snap_slot[kMaxP];
    int8_t snap_at[kMaxSteps];  // global step J: slot of the snapshot taken after J, or -1
    int8_t band_of[kMaxSteps];  // global step J: the narrowest prefix covering it (P: none)
    int32_t nslot;              // slots in use: 4 wave partials + snapshots
};

struct BwdArgs {
    const _Float16 *X16;  // outer rows scaled by their sig, FP16 [NO][D]
    const _Float16 *Y16;  // inner rows scaled by their sig, FP16 [NI][D]
    int64_t NO, NI;
    int D;
    const float *oA, *oC, *oRho;  // outer tables [P][NO]
    const float *oSig;            // outer rows' sig [NO]
    const float *iI, *iKap;       // inner tables [P][NI]: inv / sig and Kap / sig
    float b2;                     // sigmoid form: bias * log2(e)
    // operand-scale bound: U_o = sum_p wnorm_p (inv_p / inv_P)_o iyrmax_p (oNeg_p,o + gterm_p)
    const float *oInv, *oNeg;     // outer inverse norms and negative-mass fractions [P][NO] (oNeg nullable)
    const float *iyrmax;          // [P] device: max over inner rows of inv_p / sig
    const float *gterm;           // [P] device global term per prefix, or nullptr to use gterm_val
    float gterm_val[kMaxP];
    float wnorm[kMaxP];
    int64_t diag_shift;           // positive of outer o is inner (o + diag_shift) ^ pxor
    int pxor;                     // 1: one-set form, where inner o + diag_shift is o itself and is not scored
    int64_t blocks_per_split;
    int do_update, want_loss;
    float *part;   // [nsplit][NO][D]
    float *Cpart;  // [nsplit][P][NO]
    float *lossparts;
    int64_t loss_slot0;
    float *biasparts;  // sigmoid form, the pass with want_loss: [slot][P] sums of sigma(l) over the masked cells
    float *tsum;       // nullable: [NO] per outer row, sum over p of its radial coefficient (dL/dscale)
    // one inner split only: the gradient rows are finished in place (the finalize terms
    // below) and written to fin_out instead of part / Cpart
    float *fin_out;
    // listed cells: entries lent[lptr[ob] .. lptr[ob + 1]) of outer block ob (lptr nullable)
    const int32_t *lptr;
    const ListEnt *lent;
    const u16 *finX, *finY;                         // BF16 outer / inner rows
    const float *diagA, *posdot, *invx, *gam;        // as in FinArgs
    int64_t R, pos_shift;
    int accumulate;
    Prefixes pf;   // the prefix widths (generic backward)
    GenTabs gt;    // generic backward: step and slot tables of the ladder
};

struct FinArgs {
    const u16 *X, *Y;
    int64_t NO, R;
    int D;
    Prefixes pf;
    const float *part, *Cpart, *diagA, *posdot, *invx, *gam;
    int64_t nsplit, diag_shift, pos_shift;
    int pxor;  // positive's row in Y: (o + diag_shift) ^ pxor
    int accumulate;
    float *out;
    float *tsum;  // nullable: [NO] per row, sum over p of its radial coefficient (dL/dscale)
};

struct LossArgs {
    Prefixes pf;
    const float *lossparts;
    int64_t nslots;
    double norm;
    float wnorm[kMaxP];
    float *loss_out, *prefix_losses_out;
    const float *tsum;        // [ntsum] per-row radial sums of one backward pass (dL/dscale), or nullptr
    int64_t ntsum;
    float inv_scale;
    const float *biasparts;   // sigmoid form: [nslots][P] (dL/dbias), or nullptr (softmax: dL/dbias = 0)
    float *dscale_out, *dbias_out;
};

// launchers (kernels.hip)
hipError_t launch_prep(const PrepArgs &a, hipStream_t s);
// (the forward also writes posdot[p][i], the prefix dot product of row i with its positive off + i)
hipError_t launch_fwd(const u16 *q, const u16 *k, int64_t R, int64_t N, int D, const Prefixes &pf, int64_t off,
                      const float *rowA, const float *colI, float cshift, float *rowpart, float *colpart,
                      float *posdot, hipStream_t s);
hipError_t launch_rowstats(const StatsArgs &a, hipStream_t s);
hipError_t launch_colstats(const StatsArgs &a, hipStream_t s);
hipError_t launch_siglip_tabs(const StatsArgs &a, hipStream_t s);
bool bwd_mask_supported(uint32_t mask);
hipError_t launch_bwd(const BwdArgs &a, uint32_t mask, bool sig, int64_t nsplit, hipStream_t s);
// generic backward (any ladder, D <= 2048): nq = 32-wide steps per wave, a power of two <= 16
constexpr int kGenOuter = 32;  // outer rows per generic backward workgroup
int gen_max_slots(int nq);     // S slots its LDS holds at this nq
int gen_max_bands(int nq);     // band operands (prefixes + 1) its LDS holds at this nq
hipError_t launch_bwd_gen(const BwdArgs &a, int nq, bool sig, int64_t nsplit, hipStream_t s);
hipError_t launch_maxes(const float *t0, const float *t1, const float *t2, const float *t3, int64_t n0, int64_t n1,
                        int64_t n2, int64_t n3, int P, float *gmax, hipStream_t s);
hipError_t launch_finalize(const FinArgs &a, hipStream_t s);
hipError_t launch_loss(const LossArgs &a, hipStream_t s);

// Extra positives of the sigmoid form (positives.hip).  The backward passes leave every listed
// cell out (ListEnt masks); this pass gives each its positive-label loss softplus(-l) and its
// residual (sigma(l) - 1) / den = -sigma(-l) / den, all in FP32.
struct PosArgs {
    const u16 *x, *y;          // outer rows [NO][D] and inner rows [NI][D], BF16
    const float *invx, *invy;  // [P][NO], [P][NI]: 1 / |row[:w_p]|
    int64_t NO, NI;
    int D;
    Prefixes pf;
    const int32_t *ptr, *idx;  // outer row o's listed inner rows: idx[ptr[o] .. ptr[o + 1])
    float t, b;                // logit scale and bias
    float gc[kMaxP];           // mirror (w_p / W) t / den: with -sigma(-l^p), the gradient factor of a listed cell
    float *out;                // [NO][D] FP32 gradient the listed cells' terms are added to, or nullptr
    float *parts;              // [blocks][3][P]: the block's sums of softplus(-l^p), sigma(-l^p) cos^p and
                               // sigma(-l^p), or nullptr
};
struct PosFoldArgs {
    const float *parts;  // [nblk][3][P]
    int64_t nblk;
    Prefixes pf;
    double norm;         // 1 / den
    float wnorm[kMaxP];
    float *loss_out, *prefix_losses_out, *dscale_out, *dbias_out;  // updated in place (nullable but loss_out)
};
constexpr int kPosBlocks = 1024;  // most workgroups of one extra-positive pass
hipError_t launch_pos(const PosArgs &a, hipStream_t s, int64_t *blocks_out);
hipError_t launch_pos_fold(const PosFoldArgs &a, hipStream_t s);

constexpr int kFwdTile = 128;   // forward tile (rows and columns)
constexpr int kBwdOuter = 64;   // outer rows per backward workgroup
constexpr int kBwdInner = 16;   // inner rows per backward block
// rows of a backward operand copy: whole blocks plus two zero blocks, which the
// backward's copies run into past the last block
inline int64_t bwd_padded_rows(int64_t rows) { return ((rows + kBwdInner - 1) / kBwdInner + 2) * kBwdInner; }
constexpr int kStatRows = 64;   // rows per block of the statistics kernels

}  // namespace uform
