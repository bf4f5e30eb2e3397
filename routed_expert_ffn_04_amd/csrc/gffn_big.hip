// Grouped expert FFN, large tiles for groups with many rows (e4m3 and bf16).
//
// "DeepSeek V3/R1 Inference Efficiency (2)", section 2.3.1: at prefill sizes
// the routed experts see thousands of rows each ("up & gate" [7168, 4096] and
// "down" [2048, 7168] per group, FP8) and the GEMMs are compute-bound.
//
// Tile: 256 rows x 256 MFMA columns (gate/up: 128 gate + 128 up columns of
// the same 128 h columns; down: 256 output columns), K staged 128 bytes at a
// time in a double-buffered LDS ring fed by direct global->LDS 16-byte loads
// (no VGPR round trip).  LDS rows are 128 bytes with the eight 16-byte chunks
// XOR-swizzled per row (swz_key) so that fragment reads run near the LDS
// read rate.
// 8 waves (2 along M x 4 along N), each computing 128 x 64.
//   e4m3: v_mfma_scale_f32_16x16x128_f8f6f4 (unit MX scales), one per 16x16
//         block and stage: a whole 128-wide scaling block.  Its partial joins
//         the fp32 accumulator with one FMA by (activation scale x weight
//         scale); the products are formed once per row and stage in LDS.
//   bf16: v_mfma_f32_32x32x16_bf16 (the 16x16x32 form runs at half rate on
//         gfx950), four per 32x32 block and stage.
// The gate/up epilogue applies SwiGLU and quantises h per row and 128-column
// block (e4m3) or rounds it (bf16); the down epilogue writes y.
//
// Full tiles (256 rows) run a branch-free body with the A fragments
// double-buffered by name; the last, partial m-tile of a group runs a body
// that skips empty 16-row blocks.  They are separate instantiations so each
// gets its own register allocation.
//
// Tiles of a group are ordered n-tile-major with the group's m-tiles
// innermost, so the m-tiles that share a weight tile run side by side on one
// die (see TileIter) and the weight tile is read from HBM once.
#include "gffn_common.h"

namespace moe {

constexpr int kBigM = 256;        // rows per tile
constexpr int kBigN = 256;        // MFMA columns per tile
constexpr int kStage = 128;       // K bytes per stage
constexpr int kStageBytes = (kBigM + kBigN) * kStage;   // 64 KiB: A rows then B rows

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((ext_vector_type(16))) float f32x16;

// 16-byte chunk c of LDS row r sits at position c ^ key(r).  The key spreads
// both fragment shapes (16 rows x one chunk, 32 rows x one chunk) over all
// banks; measured ds_read_b128 rates on gfx950 for these shapes: ~197 B/clk
// per CU against ~118 for key (r >> 1) & 7 and ~64 unswizzled (lane-linear
// reads: ~211).
__device__ __forceinline__ int swz_key(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int swz(int row, int chunk) { return row * kStage + ((chunk ^ swz_key(row)) << 4); }

__device__ __forceinline__ const uint8_t* uniform_ptr(const void* p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return (const uint8_t*)(((uint64_t)hi << 32) | lo);
}

// The direct loads of a stage: 512 rows x 8 chunks = 4096 16-byte chunks;
// instruction q of wave w fills LDS region 8w+q (1 KiB = rows 8(8w+q) ..
// +7, lane l: row + l/8, position l%8).  Waves 0-3 move A rows, waves 4-7
// B rows, so each wave has one base address (in scalar registers); the byte
// offsets of a lane's eight chunks sit in LDS for the whole tile (registers
// are taken by the accumulators).
struct Loader {
    const uint8_t* base;   // wave-uniform
};

// Offsets of a lane's loads are kept in LDS as pairs (q even, q odd) so that
// one 8-byte read brings the two loads issued together.
__device__ __forceinline__ int loff_index(int q, int tid) { return ((q >> 1) * 512 + tid) * 2 + (q & 1); }

__device__ __forceinline__ void issue_at(uint8_t* lds_stage, const Loader& ld, uint32_t off, int k0, int wave, int q) {
    __builtin_amdgcn_global_load_lds((const void*)(ld.base + k0 + off), (lds_void*)(lds_stage + (wave * 8 + q) * 1024),
                                     16, 0, 0);
}

__device__ __forceinline__ void issue_one(uint8_t* lds_stage, const Loader& ld, const uint32_t* loff, int k0, int wave,
                                          int tid, int q) {
    issue_at(lds_stage, ld, loff[loff_index(q, tid)], k0, wave, q);
}

// 32-byte e4m3 fragment (16x16x128 operand) of the 16 rows starting at row0
// (a multiple of 16): lane l takes row row0 + l%16, bytes [32*(l/16), +32).
// The swizzle key of a row depends on its index mod 16 only, so the lane's
// two chunk offsets (Frag8Lane) are fixed and row0 becomes an immediate.
struct Frag8Lane {
    uint32_t lo, hi;
};
__device__ __forceinline__ Frag8Lane frag8_lane(int lane) {
    const int r = lane % 16, c0 = 2 * (lane / 16);
    return Frag8Lane{(uint32_t)swz(r, c0), (uint32_t)swz(r, c0 + 1)};
}
__device__ __forceinline__ i32x8 frag8(const uint8_t* base, int row0, const Frag8Lane& fl) {
    const uint8_t* p = base + row0 * kStage;
    const i32x4 lo = *(const i32x4*)(p + fl.lo);
    const i32x4 hi = *(const i32x4*)(p + fl.hi);
    return i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

// 16-byte bf16 fragment (32x32x16 operand, k-step ks of 4): row, bytes [32*ks + 16*(lane/32), +16)
__device__ __forceinline__ bf16x8 frag16(const uint8_t* base, int row, int lane, int ks) {
    return *(const bf16x8*)(base + swz(row, ks * 2 + lane / 32));
}

struct BigSmem {
    uint8_t* stage_buf;           // 2 x 64 KiB
    uint32_t* aoff;               // 256 A-row byte offsets from the A base
    int* out_row;                 // 256 output rows (-1: none)
    const float** srow;           // 256 activation-scale rows (e4m3)
    float* sprod;                 // [2 stages][256 tokens][2 kinds] scale products
    float* red;                   // [4][256] amax partials
    uint32_t* loff;               // [4][512][2] per-thread chunk offsets of the direct loads (loff_index)
};

// Promotion of one MFMA's partial products (a 16 x 16 block over a 128-wide K
// block) into the fp32 accumulators: acc += partial * (activation scale x
// weight scale).  c holds the lane's token's products with the two
// weight-scale kinds (gate/up: gate for weight blocks j < 2, up for j >= 2;
// down: the wave's 128-column block, the second one for wn >= 2).
template <int PHASE>
__device__ __forceinline__ void promote1(f32x4& acc, const f32x4& t, float2 c, int j, int wn) {
    const float cj = PHASE == 0 ? (j < 2 ? c.x : c.y) : (wn >= 2 ? c.y : c.x);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = __builtin_fmaf(t[q], cj, acc[q]);
}

// Scheduling groups of one block of the e4m3 K loop (the builtin takes
// literal arguments only; the branches fold away once the block loop is
// unrolled): nds LDS reads first, then four times one MFMA followed by four
// VALU instructions.
__device__ __forceinline__ void sched_block_order(int nds) {
    if (nds == 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
}

// One K stage of the e4m3 tile for one wave: D^T = W X^T, the MFMA row
// operand a 16-column weight block, the column operand a 16-token block; a
// lane accumulates columns 4 (l/16) + q of the weight block for token l%16.
// The wave computes its first NB 16-row token blocks (8 in full tiles; in the
// last, partial m-tile of a group the number of blocks holding rows, rounded
// up to 1, 2, 4 or 8: rows past the group's end re-read its last row and are
// never stored, so computing them is harmless).
//
// Software pipeline over the stage's MFMAs n = 4 i + j (token block i, weight
// block j): MFMA n writes its partial into T[j] of a four-deep ring, and the
// partial of MFMA n - 3 is promoted right after it is issued, so no FMA waits
// on the MFMA just issued.  The last three partials of a stage (block NB-1,
// j = 1..3) are promoted after the next stage's first MFMAs (cp: their scale
// pair).  The next block's token fragment is read one block ahead.  With MORE
// the next stage's eight direct loads of the wave go out together right after
// the stage's scale pairs and first fragments are read, so the whole stage's
// compute overlaps them (4-5% faster at T=16384 than two at a time after
// blocks 1-4); the scale pairs are read first because an 8-byte LDS read
// placed after a direct load is made to wait for it.  NB and MORE are template
// parameters so that the block sequence has no branch for the compiler to move
// the MFMAs across.
template <int PHASE, int NB, bool MORE>
__device__ __forceinline__ void fp8_stage(f32x4 (&acc8)[8][4], f32x4 (&T)[4], float2& cp, const BigSmem& S,
                                          const Loader& ld, const uint8_t* cur, uint8_t* nbuf, int k1, int s, int tid,
                                          int lane, int wave, int wm, int wn) {
    const uint8_t* As = cur;
    const uint8_t* Bs = cur + kBigM * kStage;
    const Frag8Lane fl = frag8_lane(lane);
    auto dma_pair = [&](int p) {   // loads 2p and 2p+1 of the next stage
        const uint32_t o0 = S.loff[loff_index(2 * p, tid)];
        const uint32_t o1 = S.loff[loff_index(2 * p + 1, tid)];
        issue_at(nbuf, ld, o0, k1, wave, 2 * p);
        issue_at(nbuf, ld, o1, k1, wave, 2 * p + 1);
    };
    if constexpr (NB > 0) {
        // scale pairs of this lane's token in the wave's token blocks
        const float2* sp2 = (const float2*)(S.sprod + (s & 1) * 2 * kBigM) + wm * 128 + lane % 16;
        float2 c[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) c[i] = sp2[i * 16];
        // weight blocks j: gate/up j<2 gate columns wn*32+16j, j>=2 up columns; down wn*64+16j
        i32x8 wfr[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int brow = PHASE == 0 ? (j < 2 ? wn * 32 + 16 * j : 128 + wn * 32 + 16 * (j - 2)) : wn * 64 + 16 * j;
            wfr[j] = frag8(Bs, brow, fl);
        }
        i32x8 x = frag8(As, wm * 128, fl);
        if constexpr (MORE) {
#pragma unroll
            for (int p = 0; p < 4; ++p) dma_pair(p);
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            i32x8 xn = x;
            if (i + 1 < NB) xn = frag8(As, wm * 128 + (i + 1) * 16, fl);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                T[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wfr[j], x, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0,
                                                                         127, 0, 127);
                if (j == 3)
                    promote1<PHASE>(acc8[i][0], T[0], c[i], 0, wn);
                else if (i > 0)
                    promote1<PHASE>(acc8[i - 1][j + 1], T[j + 1], c[i - 1], j + 1, wn);
                else   // the previous stage's last block (zero partials before the first stage)
                    promote1<PHASE>(acc8[NB - 1][j + 1], T[j + 1], cp, j + 1, wn);
            }
            x = xn;
            // the block's order: its LDS reads, then each MFMA followed by the
            // four promotion FMAs of the partial three MFMAs back (so the FMAs
            // run while the matrix core works)
            sched_block_order(i + 1 < NB ? 2 : 0);
            // keep the scheduler from hoisting later blocks' fragment reads
            // (register pressure: the accumulators take half the budget)
            __builtin_amdgcn_sched_barrier(0);
        }
        cp = c[NB - 1];
    }
    if constexpr (MORE && NB == 0) {
#pragma unroll
        for (int p = 0; p < 4; ++p) dma_pair(p);
    }
}

// The K loop of an e4m3 tile for a wave computing NB token blocks.  Scale
// products: activation scale of the row x weight scale of the column block,
// per row and K block, for the first (gate) and second (up) column block,
// stored per token as a (kind 0, kind 1) pair.  Stage s's products are
// written by waves 0-3 at the start of stage s-1 from scales loaded into
// registers one stage earlier (the row's activation scale by its thread, the
// two weight scales into scalar registers), so their latency hides behind a
// stage of compute; stage 0's come straight from memory at the tile start.
// (Bringing the scales in with direct-to-LDS loads instead makes the compiler
// wait for those loads before the stage's next LDS read.)  The last stage is
// peeled off the loop (it issues no loads), so the loop body is one straight
// sequence.
template <int PHASE, int NB>
__device__ __forceinline__ void fp8_kloop(f32x4 (&acc8)[8][4], const BigSmem& S, const Loader& ld, const float* wsc0,
                                          const float* wsc1, int nstages, int tid, int lane, int wave, int wm, int wn) {
    // global-address-space views: a generic load would count against the LDS
    // counter too and make the next LDS reads wait for it
    typedef const __attribute__((address_space(1))) float gfloat;
    gfloat* srow = tid < kBigM ? (gfloat*)S.srow[tid] : nullptr;
    gfloat* ws0 = (gfloat*)wsc0;
    gfloat* ws1 = (gfloat*)wsc1;
    float sa_n = 0.f, w_n0 = 0.f, w_n1 = 0.f;   // scales of the next products
    if (tid < kBigM) {
        const float sa0 = srow[0];
        ((float2*)S.sprod)[tid] = make_float2(sa0 * ws0[0], sa0 * ws1[0]);
    }
    if (1 < nstages) {
        if (tid < kBigM) sa_n = srow[1];
        w_n0 = ws0[1];
        w_n1 = ws1[1];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) issue_one(S.stage_buf, ld, S.loff, 0, wave, tid, q);

    // ring of MFMA partials and the scale pair of the last block of the
    // previous stage (zero before the first stage, so its promotion adds 0)
    f32x4 T[4] = {};
    float2 cp = make_float2(0.f, 0.f);
    // stage start: this wave's direct loads of stage s (and the scale loads
    // issued one stage earlier) landed (the barrier alone does not wait for
    // direct loads), then every wave's; stage s-1 fully consumed.  Then the
    // products of stage s+1 (into the buffer last read in stage s-1) and the
    // scale loads of stage s+2.
    auto top = [&](int s) {
        wait_vm<0>();
        __syncthreads();
        if (s + 1 < nstages) {
            if (tid < kBigM)
                ((float2*)(S.sprod + ((s + 1) & 1) * 2 * kBigM))[tid] = make_float2(sa_n * w_n0, sa_n * w_n1);
            if (s + 2 < nstages) {
                if (tid < kBigM) sa_n = srow[s + 2];
                w_n0 = ws0[s + 2];
                w_n1 = ws1[s + 2];
            }
        }
    };
    int s = 0;
    for (; s + 1 < nstages; ++s) {
        top(s);
        fp8_stage<PHASE, NB, true>(acc8, T, cp, S, ld, S.stage_buf + (s & 1) * kStageBytes,
                                   S.stage_buf + ((s + 1) & 1) * kStageBytes, (s + 1) * kStage, s, tid, lane, wave, wm,
                                   wn);
    }
    top(s);
    fp8_stage<PHASE, NB, false>(acc8, T, cp, S, ld, S.stage_buf + (s & 1) * kStageBytes, nullptr, 0, s, tid, lane,
                                wave, wm, wn);
    if constexpr (NB > 0)
#pragma unroll
        for (int j = 1; j < 4; ++j) promote1<PHASE>(acc8[NB - 1][j], T[j], cp, j, wn);
}

// One tile: K loop and epilogue.  FULL: all 256 rows hold data.
template <int DT, int PHASE, bool FULL>
__device__ __forceinline__ void big_tile(const GArgs& A, const GroupInfo& gi, const Bank& bk, const BigSmem& S,
                                         const Loader& ld, int n0, int valid, int tid, int lane, int wave, int wm, int wn) {
    constexpr bool FP8 = DT == DT_E4M3;
    constexpr int EB = FP8 ? 1 : 2;
    const int H = A.H, I = A.I;
    const int K = PHASE == 0 ? H : I;
    const int nstages = K * EB / kStage;
    // 16-row blocks of this wave that hold data
    const int nrb = FULL ? 8 : min(max((valid - wm * 128 + 15) / 16, 0), 8);

    // weight-scale rows of this tile (e4m3): gate/up: gate and up of column
    // block n0/128; down: the two 128-column blocks of the tile
    const float* wsc0 = nullptr;
    const float* wsc1 = nullptr;
    if (FP8) {
        if (PHASE == 0) {
            const size_t b = ((size_t)gi.e * (I / 128) + n0 / 128) * (H / 128);
            wsc0 = bk.sg + b;
            wsc1 = bk.su + b;
        } else {
            wsc0 = bk.sd + ((size_t)gi.e * (H / 128) + n0 / 128) * (I / 128);
            wsc1 = bk.sd + ((size_t)gi.e * (H / 128) + n0 / 128 + 1) * (I / 128);
        }
    }

    // accumulators: e4m3 16x16 blocks [8][4]; bf16 32x32 blocks [4][2]
    f32x4 acc8[FP8 ? 8 : 1][4];
    f32x16 acc16[FP8 ? 1 : 4][2];
    if (FP8) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc8[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc16[i][j] = f32x16{};
    }

    if constexpr (FP8) {
        if (FULL || nrb > 4) fp8_kloop<PHASE, 8>(acc8, S, ld, wsc0, wsc1, nstages, tid, lane, wave, wm, wn);
        else if (nrb > 2) fp8_kloop<PHASE, 4>(acc8, S, ld, wsc0, wsc1, nstages, tid, lane, wave, wm, wn);
        else if (nrb == 2) fp8_kloop<PHASE, 2>(acc8, S, ld, wsc0, wsc1, nstages, tid, lane, wave, wm, wn);
        else if (nrb == 1) fp8_kloop<PHASE, 1>(acc8, S, ld, wsc0, wsc1, nstages, tid, lane, wave, wm, wn);
        else fp8_kloop<PHASE, 0>(acc8, S, ld, wsc0, wsc1, nstages, tid, lane, wave, wm, wn);
    } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) issue_one(S.stage_buf, ld, S.loff, 0, wave, tid, q);
        // the lane's eight load offsets, the same in every stage of the tile
        uint32_t lo[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) lo[q] = S.loff[loff_index(q, tid)];
        for (int s = 0; s < nstages; ++s) {
            const uint8_t* cur = S.stage_buf + (s & 1) * kStageBytes;
            // this wave's direct loads of stage s landed (the barrier alone
            // does not wait for them), then every wave's; stage s-1 fully consumed
            wait_vm<0>();
            __syncthreads();
            // The next stage's eight direct loads of this wave are spread over
            // the compute, two after each of the first two k-steps: issued
            // back to back they would stall the wave on a full load queue (the
            // vector L1 keeps a bounded number of line misses in flight)
            // before its first MFMA.
            const bool more = s + 1 < nstages;
            uint8_t* nbuf = S.stage_buf + ((s + 1) & 1) * kStageBytes;
            const int k1 = (s + 1) * kStage;
            auto dma2 = [&](int b) {   // loads 2b and 2b+1
                if (more) {
                    issue_at(nbuf, ld, lo[2 * b], k1, wave, 2 * b);
                    issue_at(nbuf, ld, lo[2 * b + 1], k1, wave, 2 * b + 1);
                }
            };
            const uint8_t* As = cur;
            const uint8_t* Bs = cur + kBigM * kStage;
            // bf16: 32x32 blocks; B block j: gate/up j=0 gate rows wn*32.., j=1 up rows 128+wn*32..;
            // down: rows wn*64 + 32j.  The fragments of k-step ks+1 are read
            // while the MFMAs of k-step ks run (two register sets), so no
            // MFMA waits on the LDS read just issued.
            bf16x8 af[2][4], bfr[2][2];
            auto read_step = [&](int ks, bf16x8(&a)[4], bf16x8(&b)[2]) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int brow = PHASE == 0 ? (j == 0 ? wn * 32 : 128 + wn * 32) : wn * 64 + 32 * j;
                    b[j] = frag16(Bs, brow + lane % 32, lane, ks);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (FULL || 2 * i < nrb) a[i] = frag16(As, wm * 128 + i * 32 + lane % 32, lane, ks);
            };
            read_step(0, af[0], bfr[0]);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                if (ks + 1 < 4) read_step(ks + 1, af[(ks + 1) & 1], bfr[(ks + 1) & 1]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (FULL || 2 * i < nrb) {
#pragma unroll
                        for (int j = 0; j < 2; ++j)
                            acc16[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][i], bfr[ks & 1][j],
                                                                                  acc16[i][j], 0, 0, 0);
                    }
                }
                if (ks < 2) {
                    dma2(2 * ks);
                    dma2(2 * ks + 1);
                }
            }
        }
    }

    // ---------------------------------------------------------------- epilogue
    // element (i, j, v) of the wave's 128 x 64 accumulator:
    //   e4m3 16x16 (transposed): row 16 i + lane%16, col 16 j + 4 (lane/16) + v   (v < 4)
    //   bf16 32x32: row 32 i + 8 (v/4) + 4 (lane/32) + v%4, col 32 j + lane%32   (v < 16)
    if (PHASE == 0) {
        // h = silu(gate) * up for the wave's 32 h columns
        if (FP8) {
            float hv[8][2][4];
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) hv[i][j][q] = silu_mul(acc8[i][j][q], acc8[i][j + 2][q]);
            // amax over the tile's 128 h columns per row: the lane's eight,
            // the four lanes of the row (l/16), then the four wn waves
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float mx = 0.f;
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) mx = fmaxf(mx, fabsf(hv[i][j][q]));
                mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
                mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
                if (lane < 16) S.red[wn * kBigM + wm * 128 + i * 16 + lane] = mx;
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = wm * 128 + i * 16 + lane % 16;
                const int hr = S.out_row[r];
                if (hr < 0) continue;
                const float amax = fmaxf(fmaxf(S.red[r], S.red[kBigM + r]), fmaxf(S.red[2 * kBigM + r], S.red[3 * kBigM + r]));
                // the activation rule: scale amax / 448, codes h / scale (IEEE divisions)
                const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
                if (wn == 0 && lane < 16) A.h_scale[(size_t)hr * (I / 128) + n0 / 128] = sc;
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    *(uint32_t*)(A.h + (size_t)hr * I + n0 + wn * 32 + 16 * j + 4 * (lane / 16)) =
                        f32x4_to_e4m3x4(hv[i][j][0] / sc, hv[i][j][1] / sc, hv[i][j][2] / sc, hv[i][j][3] / sc);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r = wm * 128 + i * 32 + 8 * (v / 4) + 4 * (lane / 32) + v % 4;
                    const int hr = S.out_row[r];
                    if (hr < 0) continue;
                    ((uint16_t*)A.h)[(size_t)hr * I + n0 + wn * 32 + lane % 32] =
                        (uint16_t)f32_to_bf16_bits(silu_mul(acc16[i][0][v], acc16[i][1][v]));
                }
        }
    } else {
        void* yb = gi.shared ? A.y_sh : A.y;
        const int ybf = gi.shared ? A.y_sh_bf16 : A.y_bf16;
        if (FP8 && !gi.shared && A.y_e4m3) {
            // y as e4m3 per row and 128-column block (the FP8 combine): the
            // block of a row is split over waves wn and wn^1 (64 columns each)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float mx = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) mx = fmaxf(mx, fabsf(acc8[i][j][q]));
                mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
                mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
                if (lane < 16) S.red[wn * kBigM + wm * 128 + i * 16 + lane] = mx;
            }
            __syncthreads();
            const int pw = wn & ~1;   // first wave of the pair
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = wm * 128 + i * 16 + lane % 16;
                const int yr = S.out_row[r];
                if (yr < 0) continue;
                const float amax = fmaxf(S.red[pw * kBigM + r], S.red[(pw + 1) * kBigM + r]);
                // the activation rule: scale amax / 448, codes y / scale (IEEE divisions)
                const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
                if ((wn & 1) == 0 && lane < 16) A.y_scale[(size_t)yr * (H / 128) + (n0 + wn * 64) / 128] = sc;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *(uint32_t*)((uint8_t*)yb + (size_t)yr * H + n0 + wn * 64 + 16 * j + 4 * (lane / 16)) =
                        f32x4_to_e4m3x4(acc8[i][j][0] / sc, acc8[i][j][1] / sc, acc8[i][j][2] / sc,
                                        acc8[i][j][3] / sc);
            }
        } else if (FP8) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = wm * 128 + i * 16 + lane % 16;
                const int yr = S.out_row[r];
                if (yr < 0) continue;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const size_t o = (size_t)yr * H + n0 + wn * 64 + 16 * j + 4 * (lane / 16);
                    const f32x4 v = acc8[i][j];
                    if (ybf) {
                        const uint32_t lo = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
                        const uint32_t hi = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
                        *(uint2*)((uint16_t*)yb + o) = make_uint2(lo, hi);
                    } else {
                        *(f32x4*)((float*)yb + o) = v;
                    }
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r = wm * 128 + i * 32 + 8 * (v / 4) + 4 * (lane / 32) + v % 4;
                    const int yr = S.out_row[r];
                    if (yr < 0) continue;
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const size_t o = (size_t)yr * H + n0 + wn * 64 + 32 * j + lane % 32;
                        if (ybf) ((uint16_t*)yb)[o] = (uint16_t)f32_to_bf16_bits(acc16[i][j][v]);
                        else ((float*)yb)[o] = acc16[i][j][v];
                    }
                }
        }
    }
}

// PHASE 0: gate/up (+SwiGLU epilogue); PHASE 1: down.
template <int DT, int PHASE>
__global__ __launch_bounds__(512) void big_kernel(GArgs A, TileList L) {
    constexpr bool FP8 = DT == DT_E4M3;
    constexpr int EB = FP8 ? 1 : 2;
    const int H = A.H, I = A.I;
    const int K = PHASE == 0 ? H : I;                 // reduction length
    const int NOUT = PHASE == 0 ? I : H;               // output columns of the phase
    const int ncol = PHASE == 0 ? kBigN / 2 : kBigN;   // output columns per tile
    const int ntn = NOUT / ncol;

    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    BigSmem S;
    S.stage_buf = smem;
    S.aoff = (uint32_t*)(smem + 2 * kStageBytes);
    S.out_row = (int*)(S.aoff + kBigM);
    S.srow = (const float**)(S.out_row + kBigM);
    S.sprod = (float*)(S.srow + kBigM);
    S.red = S.sprod + 2 * 2 * kBigM;
    S.loff = (uint32_t*)(S.red + 4 * kBigM);

    const int tid = threadIdx.x, lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // scalar: wave-uniform branches
    const int wm = wave / 4, wn = wave % 4;

    for (TileIter it(L, ntn); it.valid(); it.next()) {
        // ---- decode: tiles of a group are n-tile-major, m-tiles innermost
        const int t = (int)it.t;
        const int eidx = t / ntn;
        const int2 ent = L.entries[eidx];
        const GroupInfo gi = group_info(A, ent.x);
        const int cg = (gi.m + kBigM - 1) / kBigM;
        const int bg = eidx - ent.y / kBigM;
        const int local = t - bg * ntn;
        const int nt = local / cg, mt = local % cg;
        const int m0 = mt * kBigM;
        const int n0 = nt * ncol;
        const int valid = min(gi.m - m0, kBigM);
        const Bank bk = gi.shared ? A.shared : A.routed;

        __syncthreads();   // previous tile is done with LDS
        if (tid < kBigM) {
            const int r = min(m0 + tid, gi.m - 1);          // rows past the end re-read the last row
            uint32_t o;
            const float* ps = nullptr;
            if (PHASE == 0) {
                int ar;
                const float* sbase;
                if (gi.shared) {
                    ar = r; sbase = A.a_sh_scale;
                } else {
                    const int pp = gi.p0 + r;
                    ar = A.src ? A.src[pp] / A.src_div : pp;
                    sbase = A.a_scale;
                }
                o = (uint32_t)ar * (uint32_t)(H * EB);
                if (FP8) ps = sbase + (size_t)ar * (H / 128);
            } else {
                const int hr = h_row(A, gi, r);
                o = (uint32_t)hr * (uint32_t)(I * EB);
                if (FP8) ps = A.h_scale + (size_t)hr * (I / 128);
            }
            S.aoff[tid] = o;
            S.srow[tid] = ps;
            S.out_row[tid] = (m0 + tid < gi.m) ? (PHASE == 0 ? h_row(A, gi, m0 + tid)
                                                             : (gi.shared ? m0 + tid : gi.p0 + m0 + tid))
                                               : -1;
        }
        __syncthreads();

        // this lane's eight chunks: LDS row 64 w + 8 q + l/8, position l%8
        Loader ld;
        if (wave < 4) {
            ld.base = uniform_ptr(PHASE == 0 ? (gi.shared ? A.a_sh : A.a) : A.h);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int row = (wave * 8 + q) * 8 + lane / 8;
                S.loff[loff_index(q, tid)] = S.aoff[row] + (uint32_t)(((lane % 8) ^ swz_key(row)) * 16);
            }
        } else {
            // gate/up: B rows 0..127 gate columns n0.., 128..255 up columns; down: columns n0..n0+255
            const void* wm_base = PHASE == 0 ? (wave < 6 ? bk.wg : bk.wu) : bk.wd;
            ld.base = uniform_ptr((const uint8_t*)wm_base + (size_t)gi.e * H * I * EB);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int row = (wave * 8 + q) * 8 + lane / 8;   // 256 .. 511
                const int j = row - kBigM;
                const int nrow = n0 + (PHASE == 0 ? (j & 127) : j);
                S.loff[loff_index(q, tid)] = (uint32_t)nrow * (uint32_t)(K * EB) + (uint32_t)(((lane % 8) ^ swz_key(row)) * 16);
            }
        }

        if (valid == kBigM) big_tile<DT, PHASE, true>(A, gi, bk, S, ld, n0, valid, tid, lane, wave, wm, wn);
        else big_tile<DT, PHASE, false>(A, gi, bk, S, ld, n0, valid, tid, lane, wave, wm, wn);
    }
}

// LDS: 2 stages + 256 A-row offsets + 256 output rows + 256 scale rows + products + amax partials
// + load offsets
constexpr size_t kBigLds = 2 * kStageBytes + kBigM * sizeof(uint32_t) + kBigM * sizeof(int) + kBigM * sizeof(void*) +
                           2 * 2 * kBigM * sizeof(float) + 4 * kBigM * sizeof(float) + 8 * 512 * sizeof(uint32_t);

template <int DT, int PHASE>
static hipError_t launch_big_t(const GArgs& A, const TileList& L, hipStream_t s) {
    static DeviceCache cache;
    const int grid = per_device(cache, [] {
        (void)hipFuncSetAttribute((const void*)big_kernel<DT, PHASE>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)kBigLds);
        return device_cu_count();   // one 512-thread workgroup per CU (LDS-limited)
    });
    hipLaunchKernelGGL((big_kernel<DT, PHASE>), dim3(grid), dim3(512), kBigLds, s, A, L);
    return hipGetLastError();
}

hipError_t launch_big_gateup(int dt, const GArgs& A, const TileList& L, hipStream_t s) {
    return dt == DT_E4M3 ? launch_big_t<DT_E4M3, 0>(A, L, s) : launch_big_t<DT_BF16, 0>(A, L, s);
}

hipError_t launch_big_down(int dt, const GArgs& A, const TileList& L, hipStream_t s) {
    return dt == DT_E4M3 ? launch_big_t<DT_E4M3, 1>(A, L, s) : launch_big_t<DT_BF16, 1>(A, L, s);
}

}  // namespace moe
