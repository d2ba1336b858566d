// k_ffn_grouped.hip -- batched-regime grouped GEMMs on FP16 MFMA (K4a, K4b)
// and the batched shared FP16 expert.
//
// Horizon RunMap "03 / Arquitetura", "04 / Resultados" (Grouped executor:
// compact experts computed in groups) and "08": compact INT4 weights with FP16
// scales are converted inside the kernel, FP16 activations, FP32 accumulation.
// With many tokens per expert the expert FFN is a dense contraction, so it
// runs on the matrix cores (v_mfma_f32_32x32x16_f16).
//
// Kernels (each described where it is defined):
//  w4_gemm_kernel       routed experts, persistent, 8 waves, every operand
//                       HBM -> LDS by direct-to-LDS loads in a 4-stage ring,
//                       INT4 weights converted to fp16(q*s) in registers;
//  f16_splitk_kernel    shared expert up to ~1024 tokens: one workgroup per
//                       (32-row tile, 64-row weight block, K part);
//  f16_dma_gemm_kernel  shared expert for larger batches: 64*RF x 128 tiles,
//                       both operands through a 3-stage direct-to-LDS ring.
//
// Scheduling: workgroups are dealt to the 8 XCDs round-robin by id
// (workgroup i runs on XCD i mod 8); each kernel maps ids so that the row
// tiles sharing a weight block (or the column tiles sharing activations) sit
// on one XCD and re-read them from its L2 instead of from HBM.
//
// Modes
//  GATEUP_W4 : A = x rows gathered through perm (token = perm[p] / k),
//              B = fused gate/up blocks, epilogue SwiGLU -> h[p][I] fp16
//  DOWN_W4   : A = h rows (sorted order), B = down blocks -> y[p][H] fp16
//  GATEUP_F16: shared expert, A = x rows, B = Wg/Wu fp16 row-major -> h fp16
//  DOWN_F16  : shared expert, A = h rows, B = Wd fp16 row-major -> out fp32
#include "k_w4_frag.h"

namespace moe {

enum { GM_GATEUP_W4 = 0, GM_DOWN_W4 = 1, GM_GATEUP_F16 = 2, GM_DOWN_F16 = 3 };

constexpr int GT = 256;       // threads per workgroup (4 waves)
constexpr int BK = 64;        // K per pipeline step
constexpr int NXCD = 8;       // XCDs of the part; workgroup i runs on XCD i mod 8

struct GemmArgs {
    const _Float16 *A;           // activations: x [T][K] or h [rows][K]
    const int32_t *perm;         // GATEUP_W4
    const int32_t *offsets;      // W4 modes: [E+1]; null for the shared expert
    const uint8_t *const *blobs; // W4 modes
    int64_t off_q, off_s;        // W4: section offsets inside a blob
    int64_t off_z;               // W4, zero-point format: zero points (scales' order, u8)
    const _Float16 *W0, *W1;     // F16 modes: gate/up or down (row-major)
    int k;                       // top-k (token = perm[p] / k)
    int E;                       // experts (1 for the shared expert)
    int rows;                    // total sorted rows (T*k) or tokens (T)
    int K;                       // reduction length (multiple of 64)
    int nblk;                    // 64-row blocks of B (output columns / 64, or I/32 fused)
    int g;                       // group size (W4)
    int ldo;                     // leading dim of the output (I for h, H for y/out)
    void *out;
    int ksw;                     // split-K kernel: workgroups sharing one output tile's K
    float *part;                 // split-K, ksw > 1: per-workgroup partial tiles
    unsigned *ctr;               // split-K, ksw > 1: arrival counter per output tile (zero)
};

// ----------------------------------------------------------------------------
// INT4 grouped GEMM with a 4-stage global->LDS pipeline (GATEUP_W4, DOWN_W4).
//
// Work item: (row tile of 32*MF sorted rows of one expert) x (512 output
// columns = eight 64-row weight blocks).  A workgroup has eight waves, two
// per SIMD, so one wave's dequantisation, LDS reads and load issue overlap
// the other's MFMAs; wave w owns weight block 8*nt + w and computes a
// 32*MF x 64 output tile (MF x 2 fragments): each dequantised weight
// fragment feeds MF MFMAs, each activation fragment two.
//
// Every operand of a 64-K step travels HBM -> LDS by the CU's direct-to-LDS
// loads (global_load_lds: each lane's bytes land at the wave's LDS base +
// lane * size), so nothing in flight occupies registers.  Per step and wave:
// 4*MF rows of the activation tile (8 rows of 128 B per 64-lane load), the
// wave's two 1 KB weight chunk runs (64 rows x 16 B) and one 4-byte load of
// the two chunks' group scales (64 rows x fp16 each).  The count is the same
// every step, so "step k has landed" is an exact vmcnt; a plain s_barrier
// then publishes it (a fence would wait for every outstanding load).
//
// Inside a step the four 16-K sub-steps are software pipelined: operands of
// sub-step s+1 (activation fragments from LDS, weights dequantised in
// registers) are fetched while the MFMAs of s run.  Before the last sub-step
// the wave holds every operand of the step, so the barrier that opens the
// next step sits there; the stage just finished is then refilled with step
// k+4.
//
// Activation stage layout: row r at r*128 B, its 16-byte piece j at slot
// j ^ f(r), f(r) = (r & 7) ^ ((r >> 3) & 1): the 8 or 16 rows one LDS pass of
// ds_read_b128 touches then hit distinct banks.
constexpr int W4_NS = 4;     // pipeline stages
constexpr int W4_WAVES = 8;  // waves per workgroup
constexpr int W4_T = W4_WAVES * 64;

template <int MF, bool ZP = false>
struct W4Stage {
    static constexpr int A = 32 * MF * 128;          // activation tile
    static constexpr int B = W4_WAVES * 2 * 1024;    // per wave: 2 chunk runs
    static constexpr int S = W4_WAVES * 256;         // per wave: [2 chunks][64 rows] fp16
    static constexpr int Z = ZP ? W4_WAVES * 128 : 0;   // per wave: [2 chunks][64 rows] u8
    static constexpr int BYTES = A + B + S + Z;
};

template <int MF, bool ZP = false>
constexpr size_t w4_lds_bytes() { return (size_t)W4_NS * W4Stage<MF, ZP>::BYTES; }

template <int PER>
__device__ __forceinline__ void wait_steps(int younger)   // younger in 0..3
{
    if (younger >= 3)
        wait_vm<3 * PER>();
    else if (younger == 2)
        wait_vm<2 * PER>();
    else if (younger == 1)
        wait_vm<PER>();
    else
        wait_vm<0>();
}
// lds_barrier (moe_common.h) waits for this wave's LDS reads only: the
// outstanding direct-to-LDS loads of later stages stay in flight.

// ----------------------------------------------------------------------------
// FP16 GEMM of the shared expert at moderate T, when (row tiles) x (4-block
// column tiles) would leave most CUs idle: one workgroup per (32-row tile,
// 64-row weight block, K part), its four waves splitting the part's K.  Both
// operands come straight from memory into the MFMA registers, 8 16-K steps in
// flight per wave (the activation rows are a few MB at most and stay in L2; a
// weight slice is read once from HBM and then from the L2 of the XCD that
// holds all its row tiles).  The waves' partial sums meet in LDS and are added
// in wave order.  With ksw > 1 K parts (few row tiles and blocks, e.g. the
// down projection at small T: 32 blocks of 64 rows for H = 2048) each
// workgroup publishes its tile with coherent stores and takes a ticket; the
// workgroup holding the last ticket adds the ksw tiles in part order (so the
// bits do not depend on arrival order), resets the counter to zero for the
// next call and runs the epilogue.
constexpr int SK_D = 8;

template <int MODE>
__global__ __launch_bounds__(GT) void f16_splitk_kernel(GemmArgs a)
{
    static_assert(MODE == GM_GATEUP_F16 || MODE == GM_DOWN_F16, "FP16 modes only");
    constexpr bool GATEUP = MODE == GM_GATEUP_F16;
    __shared__ float red[3][2][16][64];   // partials of waves 1..3

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;
    const int half = lane >> 5;
    const int R = (a.rows + 31) / 32;
    const int KSW = a.ksw;
    const int id = blockIdx.x;
    int unit, rt;   // unit = (weight block, K part)
    if ((a.nblk * KSW) % NXCD == 0) {   // all row tiles of a unit on one XCD (workgroup i -> XCD i % 8)
        const int xcd = id % NXCD, li = id / NXCD;
        unit = xcd + NXCD * (li / R);
        rt = li % R;
    } else {
        unit = id / R;
        rt = id % R;
    }
    const int blk = unit / KSW, kz = unit % KSW;
    const int p0 = rt * 32, mrows = min(32, a.rows - p0);
    const int K = a.K, KW = K / (4 * KSW);
    const int k0 = kz * (K / KSW) + wave * KW + 8 * half;
    const int nst = KW / 16;
    const _Float16 *arow = a.A + (size_t)(p0 + min(col, mrows - 1)) * K + k0;
    const _Float16 *w0, *w1;
    if constexpr (GATEUP) {
        w0 = a.W0 + (size_t)(blk * 32 + col) * K + k0;
        w1 = a.W1 + (size_t)(blk * 32 + col) * K + k0;
    } else {
        w0 = a.W0 + (size_t)(blk * 64 + col) * K + k0;
        w1 = a.W0 + (size_t)(blk * 64 + 32 + col) * K + k0;
    }
    half8_t ra[SK_D], rb0[SK_D], rb1[SK_D];
    auto load = [&](int i, int st) {   // unconditional: past the end re-reads the last step
        ra[i] = ldg(reinterpret_cast<const half8_t *>(arow + 16 * st));
        rb0[i] = ldg(reinterpret_cast<const half8_t *>(w0 + 16 * st));
        rb1[i] = ldg(reinterpret_cast<const half8_t *>(w1 + 16 * st));
    };
#pragma unroll
    for (int i = 0; i < SK_D; ++i)
        load(i, min(i, nst - 1));
    float16_t acc[2];
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[n][r] = 0.0f;
    int st = 0;
    for (; st + SK_D < nst; st += SK_D) {
#pragma unroll
        for (int i = 0; i < SK_D; ++i) {
            acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ra[i], rb0[i], acc[0], 0, 0, 0);
            acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ra[i], rb1[i], acc[1], 0, 0, 0);
            load(i, min(st + SK_D + i, nst - 1));
        }
    }
#pragma unroll
    for (int i = 0; i < SK_D; ++i) {
        if (st + i < nst) {
            acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ra[i], rb0[i], acc[0], 0, 0, 0);
            acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ra[i], rb1[i], acc[1], 0, 0, 0);
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                red[wave - 1][n][r][lane] = acc[n][r];
    }
    __syncthreads();
    // value r of lane l: token row 8*(r/4) + 4*(l/32) + (r%4), weight column l%32
    auto emit = [&](int r, float v0, float v1) {
        const int row = 8 * (r >> 2) + 4 * half + (r & 3);
        if (row >= mrows)
            return;
        const size_t p = (size_t)(p0 + row);
        if constexpr (GATEUP) {
            const float hv = v0 / (1.0f + expf(-v0)) * v1;
            static_cast<_Float16 *>(a.out)[p * a.ldo + blk * 32 + col] = (_Float16)hv;
        } else {
            static_cast<float *>(a.out)[p * a.ldo + blk * 64 + col] = v0;
            static_cast<float *>(a.out)[p * a.ldo + blk * 64 + 32 + col] = v1;
        }
    };
    if (wave == 0) {
#pragma unroll
        for (int w = 0; w < 3; ++w)
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[n][r] += red[w][n][r][lane];
    }
    if (KSW == 1) {
        if (wave != 0)
            return;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            emit(r, acc[0][r], acc[1][r]);
        return;
    }
    // K parts: publish this workgroup's tile, take a ticket; the last
    // workgroup's four waves each add rows r in [4w, 4w+4) of the ksw tiles
    // in part order and store them.
    __shared__ unsigned s_last;
    const int tile = blk * R + rt;
    float *tp = a.part + (size_t)tile * KSW * 2048;   // [ksw][2][16][64]
    if (wave == 0) {
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                __hip_atomic_store(tp + (size_t)kz * 2048 + (n * 16 + r) * 64 + lane, acc[n][r],
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);   // this wave's partial stores are acknowledged
        if (lane == 0) {
            // acquire-release at agent scope: this tile's partials are
            // visible before the counter moves, and the last workgroup reads
            // the others' partials only after their releases
            const unsigned prev = __hip_atomic_fetch_add(a.ctr + tile, 1u, __ATOMIC_ACQ_REL,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            s_last = prev == (unsigned)(KSW - 1);
        }
    }
    __syncthreads();
    if (!s_last)
        return;
    float v[2][4];
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[n][i] = 0.0f;
    for (int z = 0; z < KSW; ++z)
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v[n][i] += __hip_atomic_load(
                    tp + (size_t)z * 2048 + (n * 16 + 4 * wave + i) * 64 + lane,
                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (wave == 0 && lane == 0)
        __hip_atomic_store(a.ctr + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        emit(4 * wave + i, v[0][i], v[1][i]);
}

// ----------------------------------------------------------------------------
// FP16 GEMM of the shared expert at large T (GATEUP_F16, DOWN_F16): one
// workgroup per (row tile of 64*RF tokens) x (128 weight rows), four waves in
// a 2 x 2 grid, each owning 32*RF rows x 64 weight rows (RF x 2 fragments of
// v_mfma_f32_32x32x16_f16, tokens as the first operand).  Both operands of a
// 32-K step travel HBM -> LDS by direct-to-LDS loads in a 3-stage ring, so
// nothing in flight holds registers and two workgroups share a CU; every
// thread issues the same number of loads per step, so "step k has landed" is
// an exact vmcnt followed by a bare barrier.  Rows are 64 B (32 halfs); the
// 16-byte piece j of row r sits at slot j ^ f(r), f(r) = (r >> 2) & 3.  A
// ds_read_b128 serves 16 lanes per pass from 64 four-byte banks, and on this
// part address bit 9 also takes part in choosing the bank (measured: with
// f(r) = ((r >> 1) ^ (r >> 3)) & 3, conflict-free under the plain 64-bank
// model, the fragment reads cost two passes per 16 lanes and half the LDS
// cycles of the kernel were bank conflicts); with f(r) = (r >> 2) & 3 the
// 16 rows of a pass hit distinct banks under either mapping.
// gate/up: a tile's weight rows are 64 gate rows then the same 64 up rows, and
// wave column c takes gate fragment c and up fragment c, so each lane holds
// both halves of its SwiGLU inputs; down: 128 output columns.
constexpr int FG_BK = 32;  // K per stage

// WC wave columns: 2 (four waves, 128 weight rows, a 3-stage ring, two
// workgroups per CU) or 4 (eight waves, 256 weight rows, a 4-stage ring, one
// workgroup per CU: the same two waves per SIMD, a third fewer bytes from L2
// per MFMA and one more step in flight).
template <int WC>
constexpr int fg_stages() { return WC == 2 ? 3 : 4; }
template <int RF, int WC>
constexpr int fg_stage_bytes() { return (64 * RF + 64 * WC) * FG_BK * 2; }

template <int MODE, int RF, int WC>
__global__ __launch_bounds__(128 * WC, WC == 2 ? 2 : 1) void f16_dma_gemm_kernel(GemmArgs a)
{
    static_assert(MODE == GM_GATEUP_F16 || MODE == GM_DOWN_F16, "FP16 modes only");
    static_assert(WC == 2 || WC == 4, "four or eight waves");
    constexpr bool GATEUP = MODE == GM_GATEUP_F16;
    constexpr int NWAVE = 2 * WC;
    constexpr int NTH = 64 * NWAVE;
    constexpr int NS = fg_stages<WC>();
    constexpr int BM = 64 * RF;                    // token rows of a tile
    constexpr int BN = 64 * WC;                    // weight rows of a tile
    constexpr int A_BYTES = BM * 64;
    constexpr int STAGE = fg_stage_bytes<RF, WC>();
    constexpr int A_DMA = A_BYTES / (NTH * 16);    // 16-byte loads per thread per stage
    constexpr int B_DMA = BN * 64 / (NTH * 16);
    constexpr int PER = A_DMA + B_DMA;
    static_assert(A_DMA * NTH * 16 == A_BYTES && B_DMA * NTH * 16 == BN * 64, "stage split");
    extern __shared__ __align__(16) unsigned char smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;
    const int half = lane >> 5;
    const int wr = wave / WC, wc = wave % WC;

    const int R = (a.rows + BM - 1) / BM;
    const int NT = a.nblk / WC;
    const int id = blockIdx.x;
    int nt, rt;
    if (NT % NXCD == 0) {   // every row tile of a column tile on one XCD
        const int xcd = id % NXCD, li = id / NXCD;
        nt = xcd + NXCD * (li / R);
        rt = li % R;
    } else {
        nt = id / R;
        rt = id % R;
    }
    const int p0 = rt * BM, mrows = min(BM, a.rows - p0);
    const int K = a.K, nk = K / FG_BK;

    // load sources: load i of a wave covers 16 rows (1 KB); lane L fills slot
    // L % 4 of row L / 4, i.e. piece (L % 4) ^ f(row)
    auto fsw = [](int r) { return (r >> 2) & 3; };
    const _Float16 *asrc[A_DMA];
#pragma unroll
    for (int i = 0; i < A_DMA; ++i) {
        const int r = (i * NWAVE + wave) * 16 + (lane >> 2);
        const int j = (lane & 3) ^ fsw(r);
        asrc[i] = a.A + (size_t)(p0 + min(r, mrows - 1)) * K + j * 8;
    }
    const _Float16 *bsrc[B_DMA];
#pragma unroll
    for (int i = 0; i < B_DMA; ++i) {
        const int r = (i * NWAVE + wave) * 16 + (lane >> 2);   // weight row of the tile
        const int j = (lane & 3) ^ fsw(r);
        const _Float16 *w;
        if constexpr (GATEUP)
            w = (r < BN / 2 ? a.W0 : a.W1) + (size_t)(nt * (BN / 2) + (r & (BN / 2 - 1))) * K;
        else
            w = a.W0 + (size_t)(nt * BN + r) * K;
        bsrc[i] = w + j * 8;
    }
    auto issue = [&](int kt) {   // unconditional: past the end re-reads the last step
        const int kk = min(kt, nk - 1) * FG_BK;
        unsigned char *st = smem + (size_t)(kt % NS) * STAGE;
#pragma unroll
        for (int i = 0; i < A_DMA; ++i)
            dma16(asrc[i] + kk, st + (i * NWAVE + wave) * 1024);
#pragma unroll
        for (int i = 0; i < B_DMA; ++i)
            dma16(bsrc[i] + kk, st + A_BYTES + (i * NWAVE + wave) * 1024);
    };

    float16_t acc[RF][2];
#pragma unroll
    for (int m = 0; m < RF; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[m][n][r] = 0.0f;

    // this lane's fragment rows: A rows wr*32*RF + m*32 + col; B rows of
    // fragment n (gate/up: gate rows wc*32.., up rows 64 + wc*32..)
    const int fa = fsw(col);   // f(r) of rows congruent to col mod 32 (f depends on bits 2..3)
    auto read_frags = [&](int kt, int s, half8_t (&af)[RF], half8_t (&bf)[2]) {
        const unsigned char *st = smem + (size_t)(kt % NS) * STAGE;
        const int off = ((2 * s + half) ^ fa) << 4;
#pragma unroll
        for (int m = 0; m < RF; ++m)
            af[m] = *reinterpret_cast<const half8_t *>(st + (wr * 32 * RF + m * 32 + col) * 64 + off);
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int br = GATEUP ? n * (BN / 2) + wc * 32 + col : wc * 64 + n * 32 + col;
            bf[n] = *reinterpret_cast<const half8_t *>(st + A_BYTES + br * 64 + off);
        }
    };
    auto mfmas = [&](const half8_t (&af)[RF], const half8_t (&bf)[2]) {
#pragma unroll
        for (int m = 0; m < RF; ++m)
#pragma unroll
            for (int n = 0; n < 2; ++n)
                acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[m], bf[n], acc[m][n], 0, 0, 0);
    };
    // Software pipeline over the two 16-K sub-steps of a stage: the fragments
    // of the next sub-step are read from LDS while the MFMAs of the current
    // one run.  The barrier that opens stage kt+1 sits between the halves:
    // by then every wave holds all of stage kt in registers, so the stage is
    // refilled (with step kt + NS) right after it.
    for (int i = 0; i < NS - 1; ++i)
        issue(i);
    wait_vm<PER * (NS - 2)>();   // this wave's loads of step 0 have landed
    lds_barrier();               // everyone's have
    issue(NS - 1);
    half8_t a0[RF], b0[2], a1[RF], b1[2];
    read_frags(0, 0, a0, b0);
    for (int kt = 0; kt < nk; ++kt) {
        read_frags(kt, 1, a1, b1);
        mfmas(a0, b0);
#pragma unroll
        for (int i = 0; i < RF + 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
        }
        wait_vm<PER * (NS - 2)>();   // this wave's loads of step kt+1 have landed
        lds_barrier();               // everyone's have; stage kt is read by all
        issue(kt + NS);
        read_frags(kt + 1, 0, a0, b0);  // past the last step: the clamped re-read, unused
        mfmas(a1, b1);
#pragma unroll
        for (int i = 0; i < RF + 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    }
    wait_vm<0>();   // the ring's trailing (clamped) loads are done before the wave ends

    // value r of lane l: token row 8*(r/4) + 4*(l/32) + (r%4), weight row l%32
#pragma unroll
    for (int m = 0; m < RF; ++m) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = wr * 32 * RF + m * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            if (row >= mrows)
                continue;
            const size_t p = (size_t)(p0 + row);
            if constexpr (GATEUP) {
                const float gv = acc[m][0][r], uv = acc[m][1][r];
                const float hv = gv / (1.0f + expf(-gv)) * uv;
                static_cast<_Float16 *>(a.out)[p * a.ldo + nt * (BN / 2) + wc * 32 + col] =
                    (_Float16)hv;
            } else {
#pragma unroll
                for (int n = 0; n < 2; ++n)
                    static_cast<float *>(a.out)[p * a.ldo + nt * BN + wc * 64 + n * 32 + col] =
                        acc[m][n][r];
            }
        }
    }
}

// Per-workgroup item record (LDS): expert, row range, column tile, blob.
struct W4Item {
    int e, p0, p1, nt;
    const uint8_t *blob;
};
constexpr int W4_MAXI = 16;   // items listed per batch

template <int MF, bool ZP = false>
constexpr size_t w4_lds_total()
{
    return w4_lds_bytes<MF, ZP>() + (size_t)W4_MAXI * sizeof(W4Item) +
           (size_t)W4_MAXI * 32 * MF * sizeof(int);
}

// ZP: zero-point blobs; one more direct-to-LDS load per step and wave (4 bytes
// on lanes 0-31) brings the two chunks' zero points (64 rows x u8 each), and
// the weights are converted to fp16((u - z) s).
template <int MODE, int MF, bool ZP>
__global__ __launch_bounds__(W4_T) void w4_gemm_kernel(GemmArgs a)
{
    static_assert(MODE == GM_GATEUP_W4 || MODE == GM_DOWN_W4, "INT4 modes only");
    constexpr bool GATEUP = MODE == GM_GATEUP_W4;
    constexpr int BM = 32 * MF;
    constexpr int RPW = BM / W4_WAVES;        // activation rows loaded per wave (4*MF)
    constexpr int NA = (RPW + 7) / 8;         // their 64-lane loads (lanes 8 per row)
    constexpr int PER = NA + 3 + (ZP ? 1 : 0);   // direct-to-LDS loads per step and wave
    using St = W4Stage<MF, ZP>;

    extern __shared__ __align__(16) unsigned char smem[];
    W4Item *items = reinterpret_cast<W4Item *>(smem + (size_t)W4_NS * St::BYTES);   // [MAXI]
    int *srcs = reinterpret_cast<int *>(items + W4_MAXI);                            // [MAXI][BM]
    // expert offsets and first row tile of each expert; built in the stage
    // memory before any load targets it
    int *s_off = reinterpret_cast<int *>(smem);       // [E+1]
    int *s_ts = s_off + (a.E + 1);                    // [E+1]
    __shared__ int s_wsum[W4_WAVES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;
    const int half = lane >> 5;
    const int fcol = (col & 7) ^ ((col >> 3) & 1);   // swizzle of rows m*32 + col
    const int gshift = __builtin_ctz((unsigned)a.g);
    const int E = a.E;
    const int K = a.K;
    const int nk = K / BK;
    const int NT = (a.nblk + W4_WAVES - 1) / W4_WAVES;
    uint32_t magic;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic));

    // row tiles per expert and their exclusive scan (E <= 2 * W4_T)
    auto build_tiles = [&]() {
        const int e0 = 2 * tid;
        int c[2] = {0, 0};
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int e = e0 + i;
            if (e < E) {
                const int o = a.offsets[e];
                s_off[e] = o;
                c[i] = (a.offsets[e + 1] - o + BM - 1) / BM;
            }
        }
        if (tid == 0)
            s_off[E] = a.offsets[E];
        const int t = c[0] + c[1];
        int incl = t;
#pragma unroll
        for (int st = 1; st < 64; st <<= 1) {
            const int v = __shfl_up(incl, st, 64);
            if (lane >= st)
                incl += v;
        }
        if (lane == 63)
            s_wsum[wave] = incl;
        __syncthreads();
        int pre = 0;
        for (int w = 0; w < wave; ++w)
            pre += s_wsum[w];
        const int excl = pre + incl - t;
        if (e0 < E)
            s_ts[e0] = excl;
        if (e0 + 1 < E)
            s_ts[e0 + 1] = excl + c[0];
        if (tid == W4_T - 1)
            s_ts[E] = pre + incl;
        __syncthreads();
    };

    build_tiles();
    const int R = s_ts[E];
    const int xcd = blockIdx.x % NXCD;
    const int G = gridDim.x / NXCD;
    const int r_lo = (int)((int64_t)R * xcd / NXCD);
    const int r_hi = (int)((int64_t)R * (xcd + 1) / NXCD);
    const int nitems = (r_hi - r_lo) * NT;
    const int it0 = (int)blockIdx.x / NXCD;
    const int nmine = it0 < nitems ? (nitems - it0 + G - 1) / G : 0;

    for (int j0 = 0; j0 < nmine; j0 += W4_MAXI) {
        const int nb = min(W4_MAXI, nmine - j0);
        if (j0 > 0)
            build_tiles();   // the stages of the previous batch overwrote the table
        // ---- this batch's items: expert by binary search over the first
        // row tiles, row range, column tile, blob; then every item's source
        // rows.  All of it is read before the first load into the stages,
        // so the in-order load counter never makes a wait drain prefetches.
        if (tid < nb) {
            const int it = it0 + (j0 + tid) * G;
            const int rt = r_lo + it / NT;
            int lo = 0, hi = E - 1;   // largest e with s_ts[e] <= rt
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (s_ts[mid] <= rt)
                    lo = mid;
                else
                    hi = mid - 1;
            }
            W4Item r;
            r.e = lo;
            r.p0 = s_off[lo] + (rt - s_ts[lo]) * BM;
            r.p1 = min(s_off[lo + 1], r.p0 + BM);
            r.nt = it % NT;
            r.blob = ldg(a.blobs + lo);
            items[tid] = r;
        }
        __syncthreads();
        for (int i = tid; i < nb * BM; i += W4_T) {
            const int q = i / BM, r = i - q * BM;
            const int p0 = items[q].p0, mrows = items[q].p1 - p0;
            const int p = p0 + (r < mrows ? r : 0);   // rows past the tile re-read its first row
            srcs[i] = GATEUP ? ldg(a.perm + p) / a.k : p;
        }
        __syncthreads();

        // ---- the batch's steps as one stream: step g = item g / nk, K-step
        // g % nk, stage g % W4_NS; loads run W4_NS - 1 steps ahead, across
        // item boundaries
        const int total = nb * nk;
        int iq = 0, ikt = 0;   // next step to load
        // sources of the item being loaded (refreshed when loading moves on
        // to the next item): this lane's activation rows, weight chunk runs
        // and scale rows
        const _Float16 *asrc[NA];
        uint64_t qbase = 0, sbase = 0, zbase = 0;   // wave-uniform (scalar registers)
        auto item_sources = [&]() {
#pragma unroll
            for (int i = 0; i < NA; ++i) {
                const int r = min(wave * RPW + 8 * i + (lane >> 3), BM - 1);
                const int fr = (r & 7) ^ ((r >> 3) & 1);
                const int jp = (lane & 7) ^ fr;
                asrc[i] = a.A + (size_t)srcs[iq * BM + r] * K + jp * 8;
            }
            const int nt = __builtin_amdgcn_readfirstlane(items[iq].nt);
            const uint64_t blob = reinterpret_cast<uint64_t>(items[iq].blob);
            const uint64_t ub = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(blob >> 32)) << 32) |
                                (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)blob);
            const int bb = min(nt * W4_WAVES + wave, a.nblk - 1);
            qbase = ub + a.off_q + (uint64_t)bb * (K / 32) * 64 * 16;
            sbase = ub + a.off_s + (uint64_t)bb * (K >> gshift) * 64 * 2;
            if constexpr (ZP)
                zbase = ub + a.off_z + (uint64_t)bb * (K >> gshift) * 64;
        };
        item_sources();
        auto issue_next = [&]() {
            unsigned char *st = smem + (size_t)((iq * nk + ikt) % W4_NS) * St::BYTES;
#pragma unroll
            for (int i = 0; i < NA; ++i)
                if (8 * RPW - 64 * i >= 64 || lane < 8 * RPW - 64 * i)
                    dma16(asrc[i] + ikt * BK, st + (wave * RPW + 8 * i) * 128);
            const uint8_t *q = reinterpret_cast<const uint8_t *>(qbase) +
                               (size_t)(2 * ikt) * 1024 + lane * 16;
            dma16(q, st + St::A + wave * 2048);
            dma16(q + 1024, st + St::A + wave * 2048 + 1024);
            // lanes 0-31: chunk 2kt's group, rows 2l, 2l+1; lanes 32-63: chunk 2kt+1's
            const int grp = ((2 * ikt + half) * 32) >> gshift;
            dma4(reinterpret_cast<const uint8_t *>(sbase) + (size_t)grp * 128 + col * 4,
                 st + St::A + St::B + wave * 256);
            if constexpr (ZP) {
                // the same rows' zero points: lanes 0-15 rows 4l..4l+3 of
                // chunk 2kt, lanes 16-31 those of chunk 2kt+1 (4 bytes each)
                const int zg = ((2 * ikt + (lane >> 4)) * 32) >> gshift;
                if (lane < 32)
                    dma4(reinterpret_cast<const uint8_t *>(zbase) + (size_t)zg * 64 +
                             (lane & 15) * 4,
                         st + St::A + St::B + St::S + wave * 128);
            }
            if (++ikt == nk) {
                ikt = 0;
                if (++iq < nb)
                    item_sources();
            }
        };

        // weight words and scales of one step: fragment n = rows n*32 + col
        struct StepW {
            uint2_t q[2][2];
            f16 s[2][2];
            uint8_t z[ZP ? 2 : 1][2];
        };
        auto read_w = [&](int g, StepW &w) {
            const unsigned char *st = smem + (size_t)(g % W4_NS) * St::BYTES;
            const unsigned char *bq = st + St::A + wave * 2048;
            const unsigned char *sq = st + St::A + St::B + wave * 256;
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    w.q[n][c] = *reinterpret_cast<const uint2_t *>(bq + c * 1024 +
                                                                   (n * 32 + col) * 16 + half * 8);
                    w.s[n][c] = *reinterpret_cast<const f16 *>(sq + c * 128 + (n * 32 + col) * 2);
                    if constexpr (ZP)
                        w.z[n][c] = *(st + St::A + St::B + St::S + wave * 128 + c * 64 + n * 32 + col);
                }
        };
        auto fetch = [&](int g, int s, const StepW &w, half8_t *a_, half8_t *b_) {
            const unsigned char *st = smem + (size_t)(g % W4_NS) * St::BYTES;
#pragma unroll
            for (int m = 0; m < MF; ++m)
                a_[m] = *reinterpret_cast<const half8_t *>(
                    st + (m * 32 + col) * 128 + (((2 * s + half) ^ fcol) << 4));
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const uint2_t q = w.q[n][s >> 1];
                const f16 c = w.s[n][s >> 1];
                if constexpr (ZP) {
                    half2_t klo, khi;
                    zp_offsets(w.z[n][s >> 1], klo, khi);
                    b_[n] = dequant8_zp((s & 1) ? q.y : q.x, half2_t{c, c}, magic, klo, khi);
                } else {
                    b_[n] = dequant8((s & 1) ? q.y : q.x, half2_t{c, c}, magic);
                }
            }
        };

        float16_t acc[MF][2];
#pragma unroll
        for (int m = 0; m < MF; ++m)
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[m][n][r] = 0.0f;

        const int pre = min(W4_NS, total);
        for (int i = 0; i < pre; ++i)
            issue_next();
        wait_steps<PER>(pre - 1);
        lds_barrier();
        StepW wc, wn;
        half8_t af[2][MF], bf[2][2];
        read_w(0, wc);
        fetch(0, 0, wc, af[0], bf[0]);

        int cq = 0, ckt = 0;   // item and K-step being computed
        for (int g = 0; g < total; ++g) {
            const bool next = g + 1 < total;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if (s == 3 && next) {
                    // every operand of step g is in registers: open step g+1
                    wait_steps<PER>(min(2, total - 2 - g));
                    lds_barrier();
                }
                // weights as the 32-row operand: acc[m][n] holds C^T, so a lane
                // owns one token row and 4 consecutive output columns per
                // group of 4 values
#pragma unroll
                for (int m = 0; m < MF; ++m)
#pragma unroll
                    for (int n = 0; n < 2; ++n)
                        acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            bf[s & 1][n], af[s & 1][m], acc[m][n], 0, 0, 0);
                if (s < 3) {
                    fetch(g, s + 1, wc, af[(s + 1) & 1], bf[(s + 1) & 1]);
                } else if (next) {
                    read_w(g + 1, wn);
                    fetch(g + 1, 0, wn, af[0], bf[0]);
                    if (g + W4_NS < total)
                        issue_next();   // refills the stage of step g (read by no one now)
                }
                // issue order inside the sub-step: each of the first MF MFMAs
                // followed by one LDS operand read and three VALU ops (the
                // next sub-step's dequantisation), the rest by three VALU ops,
                // so the reads start early and the VALU work sits under the
                // matrix core (2-3% on the 64- and 512-expert layers at 4096
                // tokens against the compiler's own order)
#pragma unroll
                for (int i = 0; i < MF; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
                    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // VALU
                }
#pragma unroll
                for (int i = 0; i < MF; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
                }
            }
            if (next)
                wc = wn;
            if (++ckt < nk)
                continue;

            // ---- epilogue of item cq (the next item's first steps are already
            // loading).  acc[m][n] = (weight rows) x (tokens): value r of lane l
            // is output column 8*(r/4) + 4*(l/32) + (r%4) of fragment n and
            // token row m*32 + l%32, so r = 4j..4j+3 are 4 consecutive columns;
            // a swap between the half-waves makes them 8 (one 16-byte store;
            // 2-4% faster at 4096 tokens than 8-byte stores).
            const W4Item itm = items[cq];
            const int blk = itm.nt * W4_WAVES + wave;
            if (blk < a.nblk) {
                const int mrows = itm.p1 - itm.p0;
#pragma unroll
                for (int m = 0; m < MF; ++m) {
                    const int row = m * 32 + col;
                    // wave-uniform (the cross-lane swap below needs the
                    // whole wave): skip fragments with no row in the tile
                    if (__ballot(row < mrows) == 0ull)
                        continue;
                    // this lane's outputs of fragment f as fp16 pairs: group j
                    // (4 columns) at 8 j + 4 half.  Swapping groups 2q+1 of
                    // the lower half-wave with groups 2q of the upper one
                    // (v_permlane32_swap: lanes 32-63 of the first operand
                    // trade places with lanes 0-31 of the second) leaves each
                    // lane 8 consecutive columns at 16 q + 8 half: one
                    // 16-byte store per q instead of two 8-byte ones
                    const size_t p = (size_t)(itm.p0 + min(row, mrows - 1));
#pragma unroll
                    for (int f = 0; f < (GATEUP ? 1 : 2); ++f) {
                        uint32_t d[4][2];
#pragma unroll
                        for (int j = 0; j < 4; ++j)
#pragma unroll
                            for (int i2 = 0; i2 < 2; ++i2) {
                                half2_t v;
                                if constexpr (GATEUP) {
                                    v[0] = (_Float16)swiglu_fast(acc[m][0][4 * j + 2 * i2],
                                                                 acc[m][1][4 * j + 2 * i2]);
                                    v[1] = (_Float16)swiglu_fast(acc[m][0][4 * j + 2 * i2 + 1],
                                                                 acc[m][1][4 * j + 2 * i2 + 1]);
                                } else {
                                    v[0] = (_Float16)acc[m][f][4 * j + 2 * i2];
                                    v[1] = (_Float16)acc[m][f][4 * j + 2 * i2 + 1];
                                }
                                d[j][i2] = __builtin_bit_cast(uint32_t, v);
                            }
#pragma unroll
                        for (int q = 0; q < 2; ++q)
#pragma unroll
                            for (int i2 = 0; i2 < 2; ++i2) {
                                const auto r = __builtin_amdgcn_permlane32_swap(
                                    d[2 * q][i2], d[2 * q + 1][i2], false, false);
                                d[2 * q][i2] = r[0];
                                d[2 * q + 1][i2] = r[1];
                            }
                        if (row < mrows) {
                            _Float16 *o = static_cast<_Float16 *>(a.out) + p * a.ldo +
                                          (GATEUP ? blk * 32 : blk * 64 + f * 32) + 8 * half;
#pragma unroll
                            for (int q = 0; q < 2; ++q)
                                *reinterpret_cast<uint4_t *>(o + 16 * q) =
                                    uint4_t{d[2 * q][0], d[2 * q][1], d[2 * q + 1][0],
                                            d[2 * q + 1][1]};
                        }
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < MF; ++m)
#pragma unroll
                for (int n = 0; n < 2; ++n)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        acc[m][n][r] = 0.0f;
            ckt = 0;
            ++cq;
        }
        __syncthreads();   // stages and item lists are free for the next batch
    }
}

static int num_cus()
{
    static int n = 0;
    if (n == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            v > 0)
            n = v;
        else
            n = 256;
    }
    return n;
}

// Upper bound on row tiles: every non-empty expert adds at most one partial tile.
static int64_t tile_bound(int rows, int E, int BM)
{
    return ((int64_t)rows + BM - 1) / BM + (E > 1 ? std::min<int64_t>(E, rows) : 0);
}

// Row-tile height (32 MF rows).  Measured on the 64-expert top-8, 512-expert
// top-10 (Zipf-skewed) and 60-expert top-4 layers from 64 to 4096 tokens: up
// to 1024 rows 32-row tiles win (each workgroup has few, short items); above
// that taller tiles win even when there are fewer items than CUs, because a
// workgroup's per-item fill and epilogue dominate a short item, as long as
// they do not mostly pad: 64-row tiles while experts hold at most 40 rows on
// average (the 512-expert layer at 2560 and 10240 rows: 21-23% faster than
// 32-row tiles), 96-row tiles up to 160 (64 experts at 4096 rows: 110 us
// against 122 with 128-row and 134 with 64-row tiles; at 8192 rows 193
// against 199-200), 128-row tiles above (64 experts at 16384 and 32768 rows:
// 299 and 505 us against 313 and 519).  The one measured case off its best
// height: 60 experts at 16384 rows (128-row tiles, 6% slower than 96).
static int pick_mf(int rows, int E)
{
    if (rows <= 1024)
        return 1;
    const int64_t avg = rows / std::max(1, std::min(E, rows));
    return avg <= 40 ? 2 : (avg <= 160 ? 3 : 4);
}

// Launch of the FP16 shared-expert GEMM with RF x 2 fragments per wave and
// WC wave columns.
template <int MODE, int RF, int WC>
static int launch_fg(hipStream_t s, const GemmArgs &a)
{
    constexpr size_t lds = (size_t)fg_stages<WC>() * fg_stage_bytes<RF, WC>();
    static_assert((WC == 2 ? 2 : 1) * lds <= 160 * 1024, "workgroups per CU");
    static bool attr_set = false;   // raising the LDS limit is idempotent
    if (!attr_set) {
        hipError_t err = hipFuncSetAttribute((const void *)f16_dma_gemm_kernel<MODE, RF, WC>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (err != hipSuccess)
            return set_error(MOE_EHIP, "hipFuncSetAttribute: %s", hipGetErrorString(err));
        attr_set = true;
    }
    const int64_t grid = (((int64_t)a.rows + 64 * RF - 1) / (64 * RF)) * (a.nblk / WC);
    hipLaunchKernelGGL((f16_dma_gemm_kernel<MODE, RF, WC>), dim3((unsigned)grid), dim3(128 * WC),
                       lds, s, a);
    MOE_LAUNCH_CHECK("f16_dma_gemm_kernel");
    return MOE_OK;
}

template <int MODE, int MF, bool ZP>
static int launch_w4(hipStream_t s, const GemmArgs &a)
{
    constexpr size_t lds = w4_lds_total<MF, ZP>();
    static_assert(w4_lds_total<MF, ZP>() <= 160 * 1024, "LDS of one workgroup");
    static bool attr_set = false;   // raising the LDS limit is idempotent
    if (!attr_set) {
        hipError_t err = hipFuncSetAttribute((const void *)w4_gemm_kernel<MODE, MF, ZP>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (err != hipSuccess)
            return set_error(MOE_EHIP, "hipFuncSetAttribute: %s", hipGetErrorString(err));
        attr_set = true;
    }
    // one workgroup per CU (its LDS and eight waves fill it)
    const int64_t items = tile_bound(a.rows, a.E, 32 * MF) * ((a.nblk + W4_WAVES - 1) / W4_WAVES);
    int64_t grid = std::min<int64_t>(items, num_cus());
    grid = std::max<int64_t>(NXCD, (grid + NXCD - 1) / NXCD * NXCD);
    hipLaunchKernelGGL((w4_gemm_kernel<MODE, MF, ZP>), dim3((unsigned)grid), dim3(W4_T), lds, s,
                       a);
    MOE_LAUNCH_CHECK("w4_gemm_kernel");
    return MOE_OK;
}

constexpr int SPLITK_MAX_ROWS = 1024;   // shared expert: split-K kernel up to this many tokens
constexpr int SPLITK_TARGET_WGS = 256;   // split-K: workgroups aimed for
constexpr int SPLITK_MAX_KSW = 8;        // split-K: most K parts per output tile
// arrival counters at the front of the workspace: one per output tile of a
// launch with K parts, which has fewer than SPLITK_TARGET_WGS tiles
constexpr int SPLITK_CTR_BYTES = SPLITK_TARGET_WGS * 4 > 2048 ? SPLITK_TARGET_WGS * 4 : 2048;

// K parts per output tile: the fewest (a divisor of K/64, at most
// SPLITK_MAX_KSW, each wave keeping at least four 16-K steps) that give
// SPLITK_TARGET_WGS workgroups.  Fixed by the shape alone, so the workspace
// size does not depend on the device.
static int splitk_ksw(int rows, int K, int nblk)
{
    const int64_t tiles = (int64_t)((rows + 31) / 32) * nblk;
    const int nk = K / 64;
    int best = 1;
    for (int d = 1; d <= nk && d <= SPLITK_MAX_KSW; ++d) {
        if (nk % d)
            continue;
        if (d > 1 && nk / d < 4)
            break;
        best = d;
        if (tiles * d >= SPLITK_TARGET_WGS)
            break;
    }
    return best;
}

static bool splitk_used(int rows, int K)
{
    return rows <= SPLITK_MAX_ROWS && K % 64 == 0;
}

static size_t splitk_part_bytes(int rows, int K, int nblk)
{
    if (!splitk_used(rows, K))
        return 0;
    const int ksw = splitk_ksw(rows, K, nblk);
    return ksw > 1 ? (size_t)((rows + 31) / 32) * nblk * ksw * 2048 * sizeof(float) : 0;
}

template <int MODE, bool ZP = false>
static int launch_mode(hipStream_t s, const GemmArgs &a)
{
    if constexpr (MODE == GM_GATEUP_F16 || MODE == GM_DOWN_F16) {
        // the DMA GEMM once it has enough tiles (measured: it wins from 512
        // tokens on with I_s = 5632, from 1024 with I_s = 512)
        const int64_t fg_tiles = (((int64_t)a.rows + 127) / 128) * (a.nblk / 2);
        const bool fg = a.rows > SPLITK_MAX_ROWS || (a.rows > 256 && fg_tiles >= 64);
        if (splitk_used(a.rows, a.K) && !fg) {
            const int64_t grid = (int64_t)((a.rows + 31) / 32) * a.nblk * a.ksw;
            hipLaunchKernelGGL((f16_splitk_kernel<MODE>), dim3((unsigned)grid), dim3(GT), 0, s, a);
            MOE_LAUNCH_CHECK("f16_splitk_kernel");
            return MOE_OK;
        }
    }
    if constexpr (MODE == GM_GATEUP_W4 || MODE == GM_DOWN_W4) {
        switch (pick_mf(a.rows, a.E)) {
        case 4: return launch_w4<MODE, 4, ZP>(s, a);
        case 3: return launch_w4<MODE, 3, ZP>(s, a);
        case 2: return launch_w4<MODE, 2, ZP>(s, a);
        default: return launch_w4<MODE, 1, ZP>(s, a);
        }
    } else {
        if (a.nblk % 2 || a.K % FG_BK)
            return set_error(MOE_EUNSUPPORTED, "shared expert: sizes outside the FP16 GEMM tiles");
        // tile choice: the largest tile whose grid keeps at least 3/4 of the
        // workgroup slots busy over its rounds (256 x 256 and 128 x 256 tiles:
        // one eight-wave workgroup per CU, taken only for K >= 1024, where the
        // 4-stage ring's fill is paid back and the workgroup's LDS does not
        // keep kernels on other streams off the CU for long; 256 x 128 and
        // 128 x 128: two four-wave workgroups per CU).  Measured with 5632
        // intermediate rows: 4096 tokens 378 -> 331 us, 8192 712 -> 596 us;
        // at 2048 tokens 256 x 256 tiles (352 workgroups: a second round a
        // third full) lost 5%.
        const int64_t r4 = ((int64_t)a.rows + 255) / 256, r2 = ((int64_t)a.rows + 127) / 128;
        const int64_t cus = num_cus();
        auto fills = [&](int64_t grid, int64_t slots) {
            const int64_t rounds = (grid + slots - 1) / slots;
            return 4 * grid >= 3 * rounds * slots;
        };
        const bool wide = a.nblk % 4 == 0 && a.K >= 1024;
        if (wide && fills(r4 * (a.nblk / 4), cus))
            return launch_fg<MODE, 4, 4>(s, a);
        if (wide && fills(r2 * (a.nblk / 4), cus))
            return launch_fg<MODE, 2, 4>(s, a);
        if (r4 * (a.nblk / 2) >= 2 * cus)
            return launch_fg<MODE, 4, 2>(s, a);
        return launch_fg<MODE, 2, 2>(s, a);
    }
}

size_t ffn_batched_ws_bytes(int T, int I, int k)
{
    return (size_t)al256((int64_t)T * k * I * sizeof(_Float16));
}

int launch_ffn_batched(const void *x, const int32_t *perm, const int32_t *offsets,
                       const void *const *blobs, int T, int H, int I, int E, int k, int g,
                       int fmt, void *y, void *ws, hipStream_t s)
{
    const int rows = T * k;
    if (rows == 0)
        return MOE_OK;
    const bool zp = fmt == FMT_ZP;
    const DevLayout L = dev_layout(H, I, g, fmt);
    _Float16 *h = static_cast<_Float16 *>(ws);
    GemmArgs a{};
    a.perm = perm;
    a.offsets = offsets;
    a.blobs = reinterpret_cast<const uint8_t *const *>(blobs);
    a.k = k;
    a.E = E;
    a.rows = rows;
    a.g = g;
    // gate/up: fused 64-row blocks (I/32 of them), K = H, out h [rows][I]
    a.A = static_cast<const _Float16 *>(x);
    a.off_q = L.gu_q;
    a.off_s = L.gu_s;
    a.off_z = L.gu_z;
    a.K = H;
    a.nblk = I / 32;
    a.ldo = I;
    a.out = h;
    int rc = zp ? launch_mode<GM_GATEUP_W4, true>(s, a) : launch_mode<GM_GATEUP_W4>(s, a);
    if (rc)
        return rc;
    // down: H/64 blocks, K = I, out y [rows][H] fp16
    a.A = h;
    a.off_q = L.d_q;
    a.off_s = L.d_s;
    a.off_z = L.d_z;
    a.K = I;
    a.nblk = H / 64;
    a.ldo = H;
    a.out = y;
    return zp ? launch_mode<GM_DOWN_W4, true>(s, a) : launch_mode<GM_DOWN_W4>(s, a);
}

// Workspace of the shared expert: [arrival counters, 2 KB, zero between
// calls][h fp16 T x Is][split-K partial tiles].
size_t shared_ffn_ws_bytes(int T, int H, int Is)
{
    if (T <= 0 || Is <= 0)
        return 0;
    const size_t part = std::max(splitk_part_bytes(T, H, Is / 32), splitk_part_bytes(T, Is, H / 64));
    return SPLITK_CTR_BYTES + (size_t)al256((int64_t)T * Is * 2) + part;
}

_Float16 *shared_ffn_h(void *ws)
{
    return reinterpret_cast<_Float16 *>(static_cast<uint8_t *>(ws) + SPLITK_CTR_BYTES);
}

int launch_shared_batched(const void *x, const void *wg, const void *wu, const void *wd, int T,
                          int H, int Is, float *out, void *ws, hipStream_t s)
{
    if (T == 0)
        return MOE_OK;
    _Float16 *h = shared_ffn_h(ws);
    GemmArgs a{};
    a.E = 1;
    a.rows = T;
    a.A = static_cast<const _Float16 *>(x);
    a.W0 = static_cast<const _Float16 *>(wg);
    a.W1 = static_cast<const _Float16 *>(wu);
    a.K = H;
    a.nblk = Is / 32;
    a.ldo = Is;
    a.out = h;
    a.ctr = static_cast<unsigned *>(ws);
    a.part = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(h) + al256((int64_t)T * Is * 2));
    a.ksw = splitk_ksw(a.rows, a.K, a.nblk);
    if (a.ksw > 1 && (int64_t)((T + 31) / 32) * a.nblk * 4 > SPLITK_CTR_BYTES)
        return set_error(MOE_EUNSUPPORTED, "shared expert: too many split-K tiles");
    int rc = launch_mode<GM_GATEUP_F16>(s, a);
    if (rc)
        return rc;
    a.A = h;
    a.W0 = static_cast<const _Float16 *>(wd);
    a.W1 = nullptr;
    a.K = Is;
    a.nblk = H / 64;
    a.ldo = H;
    a.out = out;
    a.ksw = splitk_ksw(a.rows, a.K, a.nblk);
    if (a.ksw > 1 && (int64_t)((T + 31) / 32) * a.nblk * 4 > SPLITK_CTR_BYTES)
        return set_error(MOE_EUNSUPPORTED, "shared expert: too many split-K tiles");
    return launch_mode<GM_DOWN_F16>(s, a);
}

}  // namespace moe
