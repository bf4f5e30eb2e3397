// Grouped expert FFN with MXFP4 expert weights (OCP Microscaling: E2M1
// codes, two per byte, with one E8M0 exponent per 32 consecutive reduction
// elements) and MXFP8 activations (E4M3 codes with E8M0 per 32).
//
// The pages run the MoE GEMMs of their Blackwell deployment in FP4 ("How
// DeepSeek inference works", the FP8/FP4 lever of its deployment table; "The
// 31-Millisecond Smoking Gun", the FP4 MoE backends): in the decode regime the
// grouped GEMM streams every touched expert's weights once, so 4.25 bits per
// weight instead of 8 (or 16) cuts the dominant HBM traffic.  gfx950 consumes
// both formats natively: v_mfma_scale_f32_16x16x128_f8f6f4 multiplies a
// 16 x 128 FP8 tile by a 128 x 16 FP4 tile and applies one E8M0 exponent per
// lane and 32-element K block to each operand, which is exactly the MX block.
//
// Operand layout of one MFMA (16 rows x 16 columns x 128 K), as measured on
// gfx950 with one-hot operands: lane l serves row (or column) l % 16 with
// lane group g = l / 16, and
//   FP4 weight:      K 32g .. 32g+31 (16 bytes, lower K in the low nibble);
//   FP8 activation:  K 16g .. 16g+15 (bytes 0-15) and 64+16g .. 64+16g+15
//                    (bytes 16-31);
//   E8M0 exponents:  the block of K 32g .. 32g+31 of both operands.
// The weight operand is 16 contiguous bytes of an output-major weight row and
// the activation operand two 16-byte pieces of a row, so both can be read
// from memory straight into registers (the weight never touches LDS); the
// exponents of a step's four K blocks are one dword, from which each lane
// shifts out its own byte.  The 16-row gate/up tiles instead bring the
// tile's activation rows and their exponents into LDS once per tile with
// direct loads (all four waves read the same rows at every step, which as
// register loads cost more than the weights' own share of the load path).
//
// Like the bf16 streaming kernels (gffn_stream.hip): tiles of MB*16 rows x TN
// columns x all of K, P k-steps of loads in flight per wave, waves split K
// (KS) or N, partial sums meet in LDS.  The gate/up epilogue applies SwiGLU
// and writes h as MXFP8 along I (the down projection's activation), the down
// epilogue writes fp32 or bf16 outputs.  Rows past a group's end re-read its
// last row and are never stored.
#include "gffn_common.h"

namespace moe {

namespace {


// A load through the constant address space, for data no kernel of the
// launch writes: at a wave-uniform address the compiler makes it a scalar load.
template <class T>
__device__ __forceinline__ T cld(const void* p) {
    return *(const __attribute__((address_space(4))) T*)p;
}

__device__ __forceinline__ i32x8 widen(i32x4 v) { return i32x8{v.x, v.y, v.z, v.w, 0, 0, 0, 0}; }

// Loads through global-address-space pointers: every operand lives in device
// memory, and a load the compiler cannot place (a generic "flat" access)
// would also count against the LDS counter and force full waits in the
// software pipeline.
template <class T>
__device__ __forceinline__ T gld(const uint8_t* p) {
    return *(const __attribute__((address_space(1))) T*)p;
}

// The activation operand of lane group g: p = row + step K offset + 16 g;
// bytes 0-15 from p, bytes 16-31 from p + 64.  Tile rows past the group's
// end re-read its last row (their outputs are never stored); in the decode
// regime most of a tile's 16 rows are such repeats, which cost little
// (measured: masking them off with zero-filling buffer loads was slower).
__device__ __forceinline__ i32x8 load_act(const uint8_t* p) {
    const i32x4 lo = gld<i32x4>(p), hi = gld<i32x4>(p + 64);
    return i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

// Exponents in 16-step blocks: a lane of lane group g loads the 16 bytes of
// its row's exponents for steps 4g .. 4g+3 of the block (one dword per step,
// one byte per K block of the step), and at step s of the block a lane takes
// dword s % 4 of lane group s / 4 of its row by a cross-lane read
// (ds_bpermute), then shifts out its own byte.  One 16-byte load per stream
// and 16 steps instead of a dword per step: the exponent loads had cost the
// streaming kernels 10-15% of their time.
__device__ __forceinline__ uint32_t xlane(int src_lane, int v) {
    return (uint32_t)__builtin_amdgcn_ds_bpermute(src_lane << 2, v);
}

// D += A(fp8, exponents ea) x B(fp4, exponents eb); the low byte of ea / eb
// is this lane's E8M0 (operand formats: 0 = FP8 E4M3, 4 = FP4 E2M1).
__device__ __forceinline__ f32x4 mma_f8f4(i32x8 a, i32x4 b, f32x4 c, uint32_t ea, uint32_t eb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, widen(b), c, 0, 4, 0, (int)ea, 0, (int)eb);
}

// Row of the activation matrix that tile row r (< gi.m) reads in the gate/up phase.
__device__ __forceinline__ long act_row(const GArgs& A, const GroupInfo& gi, int r) {
    if (gi.shared) return r;
    const int pp = gi.p0 + r;
    return A.src ? A.src[pp] / A.src_div : pp;
}

}  // namespace

// ---------------------------------------------------------------- gate / up
template <int MB, int KS, int P, int kNB, bool XEX, bool LDSA = false, bool XP = false>
__global__ __launch_bounds__(256) void mx_gateup_kernel(GArgs A, TileList L) {
    static_assert(!LDSA || (MB == 1 && KS == 1 && !XEX), "activations in LDS: 16-row tiles, all of K per wave, "
                                                         "exponent dwords per step");
    static_assert(!XP || (LDSA && kNB == 2 && P % 4 == 0), "packed exponents: four weight blocks per wave");
    constexpr int NW = 4 / KS;                 // waves along N
    constexpr int TN = NW * kNB * 16;          // h columns per tile (a multiple of 32)
    constexpr int RS = 2 * TN + 1;
    const int H = A.H, I = A.I;
    const int ntn = I / TN;
    const int nsteps = H / 128 / KS;           // k-steps of 128 per wave

    __shared__ float red[KS][16 * MB][RS];
    // LDSA: the tile's 16 activation rows [16][H + 16] (codes; the 16 spare
    // bytes per row spread the rows over the LDS banks), then their exponent
    // rows [16][H/32 + 4]
    extern __shared__ __attribute__((aligned(16))) uint8_t act_lds[];
    const int astride = H + 16, estride = H / 32 + 4;
    const uint8_t* exp_lds = act_lds + 16 * astride;

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int kw = wave % KS, nw = wave / KS;
    const int kq = lane / 16;                  // K block of this lane within a step
    const uint32_t esh = 8u * kq;              // its exponent byte within the step's dword
    constexpr bool XE = XEX && P % 4 == 0 && 16 % P == 0;   // exponents in 16-step blocks

    for (TileIter it(L, ntn); it.valid(); it.next()) {
        const int t = (int)it.t;
        __syncthreads();   // the previous tile's epilogue is done with `red`
        const int2 tc = tile_coords<MB == 1>(L, t, ntn);
        const int2 tl = L.entries[tc.x];
        const GroupInfo gi = group_info(A, tl.x);
        const int m0 = tl.y;
        const int nt0 = tc.y * TN;
        const int n0 = nt0 + nw * kNB * 16;
        const Bank bk = gi.shared ? A.shared : A.routed;
        const int k0 = kw * nsteps * 128;

        const uint8_t* abase = gi.shared ? A.a_sh : A.a;
        const uint8_t* aebase = (const uint8_t*)(gi.shared ? A.a_sh_scale : A.a_scale);
        if constexpr (LDSA) {
            // the tile's rows (rows past the group's end: its last row) by
            // direct loads, wave w rows 4w..4w+3, once per tile
#pragma unroll 1
            for (int rr = 0; rr < 4; ++rr) {
                const int row = 4 * wave + rr;
                const long ar = act_row(A, gi, min(m0 + row, gi.m - 1));
                const uint8_t* src = abase + (size_t)ar * H;
                const uint8_t* esrc = aebase + (size_t)ar * (H / 32);
                uint8_t* dst = act_lds + row * astride;
                uint8_t* edst = (uint8_t*)exp_lds + row * estride;
                for (int c = 0; c < H; c += 1024)
                    if (c + lane * 16 < H)
                        __builtin_amdgcn_global_load_lds((const void*)(src + c + lane * 16),
                                                         (__attribute__((address_space(3))) void*)(dst + c), 16, 0, 0);
                for (int c = 0; c < H / 32; c += 256)
                    if (c + lane * 4 < H / 32)
                        __builtin_amdgcn_global_load_lds((const void*)(esrc + c + lane * 4),
                                                         (__attribute__((address_space(3))) void*)(edst + c), 4, 0, 0);
            }
            wait_vm<0>();
            __syncthreads();
        }
        const uint8_t* ap[MB];
        const uint8_t* aep[MB];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            const long ar = act_row(A, gi, min(m0 + i * 16 + lane % 16, gi.m - 1));
            ap[i] = abase + (size_t)ar * H + k0 + kq * 16;
            aep[i] = aebase + (size_t)ar * (H / 32) + k0 / 32;
        }
        const uint8_t *gp[kNB], *up[kNB], *gep[kNB], *uep[kNB];
#pragma unroll
        for (int c = 0; c < kNB; ++c) {
            const size_t row = (size_t)gi.e * I + n0 + c * 16 + lane % 16;
            gp[c] = (const uint8_t*)bk.wg + row * (H / 2) + (k0 + kq * 32) / 2;
            up[c] = (const uint8_t*)bk.wu + row * (H / 2) + (k0 + kq * 32) / 2;
            gep[c] = (const uint8_t*)bk.sg + row * (H / 32) + k0 / 32;
            uep[c] = (const uint8_t*)bk.su + row * (H / 32) + k0 / 32;
        }
        // XP: the packed exponents of the wave's four weight blocks (gate 0,
        // gate 1, up 0, up 1), 1 KiB per four steps: one 16-byte load per
        // lane brings its own bytes of all four blocks
        const uint8_t* xpp = XP ? bk.xgu + (((size_t)gi.e * (I / 32) + n0 / 32) * (H / 512)) * 1024 + lane * 16 : nullptr;
        i32x4 xpv[P / 4 > 0 ? P / 4 : 1];

        f32x4 accg[MB][kNB], accu[MB][kNB];
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int c = 0; c < kNB; ++c) accg[i][c] = accu[i][c] = f32x4{0.f, 0.f, 0.f, 0.f};

        i32x8 ra[P][MB];
        uint32_t rae[P][MB];
        i32x4 rg[P][kNB], ru[P][kNB];
        uint32_t rge[P][kNB], rue[P][kNB];
        // exponent blocks (XE): current and next 16 steps
        i32x4 xcg[kNB], xcu[kNB], xca[MB], xng[kNB], xnu[kNB], xna[MB];
        auto load_w = [&](int p, int step) {
#pragma unroll
            for (int c = 0; c < kNB; ++c) {
                rg[p][c] = gld<i32x4>(gp[c] + step * 64);
                ru[p][c] = gld<i32x4>(up[c] + step * 64);
            }
            if constexpr (!LDSA) {
#pragma unroll
                for (int i = 0; i < MB; ++i) ra[p][i] = load_act(ap[i] + step * 128);
            }
        };
        auto load_e = [&](int p, int step) {
            if constexpr (XP) {
                // steps step-3 .. step, once step p - 3 .. p of this ring slot group are consumed
                if ((p & 3) == 3) xpv[p >> 2] = gld<i32x4>(xpp + (size_t)((step - 3) >> 2) * 1024);
                return;
            }
#pragma unroll
            for (int c = 0; c < kNB; ++c) {
                rge[p][c] = gld<uint32_t>(gep[c] + step * 4);
                rue[p][c] = gld<uint32_t>(uep[c] + step * 4);
            }
            if constexpr (!LDSA) {
#pragma unroll
                for (int i = 0; i < MB; ++i) rae[p][i] = gld<uint32_t>(aep[i] + step * 4);
            }
        };
        auto load_x = [&](int blk, i32x4 (&xg)[kNB], i32x4 (&xu)[kNB], i32x4 (&xa)[MB]) {
#pragma unroll
            for (int c = 0; c < kNB; ++c) {
                xg[c] = gld<i32x4>(gep[c] + blk * 64 + kq * 16);
                xu[c] = gld<i32x4>(uep[c] + blk * 64 + kq * 16);
            }
            if constexpr (!LDSA) {
#pragma unroll
                for (int i = 0; i < MB; ++i) xa[i] = gld<i32x4>(aep[i] + blk * 64 + kq * 16);
            }
        };
        auto next_block = [&]() {
#pragma unroll
            for (int c = 0; c < kNB; ++c) {
                xcg[c] = xng[c];
                xcu[c] = xnu[c];
            }
            if constexpr (!LDSA) {
#pragma unroll
                for (int i = 0; i < MB; ++i) xca[i] = xna[i];
            }
        };
        // step p of the ring; s0 (a multiple of 4 when XE) is the ring's first step
        auto mma = [&](int p, int s0, bool x) {
            uint32_t ea[MB], eg[kNB], eu[kNB];
            i32x8 av[MB];
            if constexpr (LDSA) {
                // lane group kq: bytes 16 kq .. +15 and 64 + 16 kq .. +15 of the step's 128
                const uint8_t* q = act_lds + (lane % 16) * astride + (s0 + p) * 128 + kq * 16;
                const i32x4 lo = *(const i32x4*)q, hi = *(const i32x4*)(q + 64);
                av[0] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            } else {
#pragma unroll
                for (int i = 0; i < MB; ++i) av[i] = ra[p][i];
            }
            if (x) {
                const int src = (lane & 15) + 16 * (((s0 + p) & 15) >> 2);
#pragma unroll
                for (int c = 0; c < kNB; ++c) {
                    eg[c] = xlane(src, xcg[c][p & 3]) >> esh;
                    eu[c] = xlane(src, xcu[c][p & 3]) >> esh;
                }
                if constexpr (!LDSA) {
#pragma unroll
                    for (int i = 0; i < MB; ++i) ea[i] = xlane(src, xca[i][p & 3]) >> esh;
                }
            } else {
                if constexpr (XP) {
                    const uint32_t v = (uint32_t)xpv[p >> 2][p & 3];
#pragma unroll
                    for (int c = 0; c < kNB; ++c) {
                        eg[c] = v >> (8 * c);
                        eu[c] = v >> (8 * (2 + c));
                    }
                } else {
#pragma unroll
                    for (int c = 0; c < kNB; ++c) {
                        eg[c] = rge[p][c] >> esh;
                        eu[c] = rue[p][c] >> esh;
                    }
                }
                if constexpr (!LDSA) {
#pragma unroll
                    for (int i = 0; i < MB; ++i) ea[i] = rae[p][i] >> esh;
                }
            }
            if constexpr (LDSA) ea[0] = *(const uint32_t*)(exp_lds + (lane % 16) * estride + (s0 + p) * 4) >> esh;
#pragma unroll
            for (int c = 0; c < kNB; ++c)
#pragma unroll
                for (int i = 0; i < MB; ++i) {
                    accg[i][c] = mma_f8f4(av[i], rg[p][c], accg[i][c], ea[i], eg[c]);
                    accu[i][c] = mma_f8f4(av[i], ru[p][c], accu[i][c], ea[i], eu[c]);
                }
        };
        // ring of P k-steps in flight over the largest multiple of P (of 16
        // with XE), then the remaining steps one at a time.  The compiler
        // gathers the refill loads at the end of each ring and counts its
        // waits per step; scheduling barriers that pin each refill behind its
        // step's MFMAs were measured ~40% slower.
        const int nmain = XE ? nsteps / 16 * 16 : nsteps / P * P;
        if (nmain > 0) {
            if (XE) {
                load_x(0, xcg, xcu, xca);
                if (nmain > 16) load_x(1, xng, xnu, xna);
            }
#pragma unroll
            for (int p = 0; p < P; ++p) {
                load_w(p, p);
                if (!XE) load_e(p, p);
            }
            int s0 = 0;
            for (; s0 < nmain - P; s0 += P) {
                if (XE && s0 > 0 && (s0 & 15) == 0) {
                    next_block();
                    if (s0 + 16 < nmain) load_x(s0 / 16 + 1, xng, xnu, xna);
                }
#pragma unroll
                for (int p = 0; p < P; ++p) {
                    mma(p, s0, XE);
                    load_w(p, s0 + P + p);
                    if (!XE) load_e(p, s0 + P + p);
                }
            }
            if (XE && s0 > 0 && (s0 & 15) == 0) next_block();
#pragma unroll
            for (int p = 0; p < P; ++p) mma(p, s0, XE);
        }
        for (int s = nmain; s < nsteps; ++s) {
            load_w(0, s);
            load_e(0, s);
            mma(0, s, false);
        }

        // partial sums -> LDS; row = i*16 + 4*(lane/16) + q, col = nw*32 + c*16 + lane%16
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int c = 0; c < kNB; ++c)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int row = i * 16 + 4 * (lane / 16) + q;
                    const int col = nw * kNB * 16 + c * 16 + lane % 16;
                    red[kw][row][col] = accg[i][c][q];
                    red[kw][row][TN + col] = accu[i][c][q];
                }
        __syncthreads();
        // SwiGLU, then MXFP8 along I: a thread takes 4 adjacent columns, so
        // the 8 threads of one 32-column block are 8 adjacent lanes (TN is a
        // multiple of 32 and the loop bound a multiple of 8: whole blocks
        // enter or leave the loop together).
        constexpr int TQ = TN / 4;
        uint8_t* he = (uint8_t*)A.h_scale;
        for (int e = tid; e < 16 * MB * TQ; e += 256) {
            const int row = e / TQ, c4 = (e % TQ) * 4;
            float hv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float g = 0.f, u = 0.f;
#pragma unroll
                for (int w = 0; w < KS; ++w) {
                    g += red[w][row][c4 + j];
                    u += red[w][row][TN + c4 + j];
                }
                hv[j] = silu_mul(g, u);
            }
            float amax = fmaxf(fmaxf(fabsf(hv[0]), fabsf(hv[1])), fmaxf(fabsf(hv[2]), fabsf(hv[3])));
            amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
            amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
            amax = fmaxf(amax, __shfl_xor(amax, 4, kWave));
            const uint32_t E = mx_e8m0_for_e4m3(amax);
            const float f = mx_inv_scale(E);
            const uint32_t code = f32x4_to_e4m3x4(hv[0] * f, hv[1] * f, hv[2] * f, hv[3] * f);
            const int r = m0 + row;
            if (r < gi.m) {
                const int hr = h_row(A, gi, r);
                *(uint32_t*)(A.h + (size_t)hr * I + nt0 + c4) = code;
                if ((c4 & 31) == 0) he[(size_t)hr * (I / 32) + (nt0 + c4) / 32] = (uint8_t)E;
            }
        }
    }
}

// ---------------------------------------------------------------- gate / up, tiles overlapped
// Workgroup barrier once this wave's LDS operations have completed, leaving
// its vector-memory operations in flight (__syncthreads would wait for them).
__device__ __forceinline__ void barrier_lds() {
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));   // vmcnt 63: no wait; lgkmcnt 0
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// The 16-row gate/up tiles of banks with packed exponents (activation rows
// in LDS, two 16-column blocks of gate and of up per wave, P k-steps of
// weights in flight), with consecutive tiles of a workgroup overlapped.  The
// next tile's set-up (tile list, group offsets, its rows' src entries) is
// done at the start of the current tile; the last P k-steps refill the ring
// with the next tile's first P, and the next tile's activation rows are
// loaded into LDS right after the epilogue's first barrier (every wave is
// past its last multiply then).  A tile thus starts with its rows and first
// weights in flight since the previous epilogue, where it used to look up
// its rows, load them, wait for them, and only then start its weight
// stream.  (Loading the rows' first columns earlier, during the last P
// k-steps, gains nothing: the compiler cannot count the direct loads of a
// loop of runtime length, so the next multiply would wait for them.)
// H / 128 is a multiple of P and at least 2 P.
template <int P, int NWV>
__global__ __launch_bounds__(64 * NWV) void mx_gateup_ovl_kernel(GArgs A, TileList L) {
    static_assert(P % 4 == 0, "one packed exponent record per four k-steps");
    constexpr int kNB = 2;
    static_assert(NWV == 4 || NWV == 8, "four or eight waves");
    constexpr int NT = 64 * NWV;               // threads
    constexpr int RW = 16 / NWV;               // activation rows loaded per wave
    constexpr int TN = NWV * kNB * 16;         // h columns per tile
    constexpr int RS = 2 * TN + 1;
    const int H = A.H, I = A.I;
    const int ntn = I / TN;
    const int nsteps = H / 128;

    __shared__ float red[16][RS];
    extern __shared__ __attribute__((aligned(16))) uint8_t act_lds[];
    const int astride = H + 16, estride = H / 32 + 4;
    uint8_t* exp_lds = act_lds + 16 * astride;

    const int tid = threadIdx.x, lane = tid % kWave;
    // wave-uniform: the next tile's row lookups are then scalar loads, which
    // do not wait behind the vector loads in flight
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int kq = lane / 16;
    const uint32_t esh = 8u * kq;

    struct Tile {
        GroupInfo gi;
        int m0, nt0;
        int nrows;                             // the tile's rows within its group (1 .. 16)
        const uint8_t *gp[kNB], *up[kNB], *xpp;
        const uint8_t *arow[RW], *erow[RW];    // this wave's activation rows and their exponents
    };
    // The next tile's set-up runs with the current tile's loads in flight.
    // Its lookups (tile list, group offsets, src rows: written by earlier
    // kernels, only read here) go through the constant address space, so
    // that at wave-uniform addresses they are scalar loads: a vector load
    // there would make the wave wait for every load issued before it.
    auto setup = [&](long t, Tile& q) {
        const int cnt = cld<int>(L.count);
        const int* ent = (const int*)(L.entries + t % cnt);   // n-major order, as tile_coords<true>
        const int2 tl = make_int2(cld<int>(ent), cld<int>(ent + 1));
        const int g = tl.x;
        if (g < A.G) {
            q.gi.p0 = min(max(cld<int>(A.offsets + g), 0), A.R_max);
            q.gi.m = min(max(cld<int>(A.offsets + g + 1) - q.gi.p0, 0), A.R_max - q.gi.p0);
            q.gi.e = g;
            q.gi.shared = 0;
        } else {
            q.gi.p0 = 0;
            q.gi.m = A.S;
            q.gi.e = 0;
            q.gi.shared = 1;
        }
        q.m0 = tl.y;
        q.nrows = min(16, q.gi.m - q.m0);
        q.nt0 = (int)(t / cnt) * TN;
        const int n0 = q.nt0 + wave * kNB * 16;
        const Bank bk = q.gi.shared ? A.shared : A.routed;
        const uint8_t* abase = q.gi.shared ? A.a_sh : A.a;
        const uint8_t* aebase = (const uint8_t*)(q.gi.shared ? A.a_sh_scale : A.a_scale);
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) {
            const int r = min(q.m0 + RW * wave + rr, q.gi.m - 1);
            const long ar = q.gi.shared ? r : A.src ? cld<int>(A.src + q.gi.p0 + r) / A.src_div : q.gi.p0 + r;
            q.arow[rr] = abase + (size_t)ar * H;
            q.erow[rr] = aebase + (size_t)ar * (H / 32);
        }
#pragma unroll
        for (int c = 0; c < kNB; ++c) {
            const size_t row = (size_t)q.gi.e * I + n0 + c * 16 + lane % 16;
            q.gp[c] = (const uint8_t*)bk.wg + row * (H / 2) + kq * 16;
            q.up[c] = (const uint8_t*)bk.wu + row * (H / 2) + kq * 16;
        }
        q.xpp = bk.xgu + (((size_t)q.gi.e * (I / 32) + n0 / 32) * (H / 512)) * 1024 + lane * 16;
    };
    // activation columns [k0, k1) and their exponents of this wave's rows, by
    // direct loads (kept behind the refill loads, which the last multiplies
    // wait for).  Only the tile's rows within its group are loaded: the
    // multiplies read row min(r, nrows - 1) for the rows past it, whose
    // outputs are never stored (a decode tile holds a few rows of 16).
    auto load_rows = [&](const Tile& q, int k0, int k1) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rr = 0; rr < RW; ++rr) {
            const int row = RW * wave + rr;
            if (row >= q.nrows) break;
            uint8_t* dst = act_lds + row * astride;
            for (int c = k0; c < k1; c += 1024)
                if (c + lane * 16 < k1)
                    __builtin_amdgcn_global_load_lds((const void*)(q.arow[rr] + c + lane * 16),
                                                     (__attribute__((address_space(3))) void*)(dst + c), 16, 0, 0);
            uint8_t* edst = exp_lds + row * estride;
            for (int c = k0 / 32; c < k1 / 32; c += 256)
                if (c + lane * 4 < k1 / 32)
                    __builtin_amdgcn_global_load_lds((const void*)(q.erow[rr] + c + lane * 4),
                                                     (__attribute__((address_space(3))) void*)(edst + c), 4, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    i32x4 rg[P][kNB], ru[P][kNB];
    i32x4 xpv[P / 4];
    f32x4 accg[kNB], accu[kNB];
    // the refill of the whole ring with k-steps step0 .. step0 + P - 1, once
    // its last multiply is issued: the exponent records first, then the
    // weights.  Scheduling barriers keep that order and the multiplies
    // above; with the records last, the compiler hoisted their exponent
    // shifts to the ring's second multiply, which then waited for every load.
    auto refill = [&](int step0, const Tile& q) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int g = 0; g < P / 4; ++g) xpv[g] = gld<i32x4>(q.xpp + (size_t)(step0 / 4 + g) * 1024);
#pragma unroll
        for (int p = 0; p < P; ++p)
#pragma unroll
            for (int c = 0; c < kNB; ++c) {
                rg[p][c] = gld<i32x4>(q.gp[c] + (step0 + p) * 64);
                ru[p][c] = gld<i32x4>(q.up[c] + (step0 + p) * 64);
            }
        __builtin_amdgcn_sched_barrier(0);
    };
    int arow_lds = 0;                          // this lane's LDS row: min(lane % 16, nrows - 1)
    auto mma = [&](int p, int step) {
        const uint8_t* qa = act_lds + arow_lds * astride + step * 128 + kq * 16;
        const i32x4 lo = *(const i32x4*)qa, hi = *(const i32x4*)(qa + 64);
        const i32x8 av = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        const uint32_t ea = *(const uint32_t*)(exp_lds + arow_lds * estride + step * 4) >> esh;
        const uint32_t v = (uint32_t)xpv[p >> 2][p & 3];
#pragma unroll
        for (int c = 0; c < kNB; ++c) {
            accg[c] = mma_f8f4(av, rg[p][c], accg[c], ea, v >> (8 * c));
            accu[c] = mma_f8f4(av, ru[p][c], accu[c], ea, v >> (8 * (2 + c)));
        }
    };

    TileIter it(L, ntn);
    if (!it.valid()) return;
    Tile cur;
    setup(it.t, cur);
    load_rows(cur, 0, H);
    refill(0, cur);
    wait_vm<0>();
    barrier_lds();
    for (;;) {
        arow_lds = min(lane % 16, cur.nrows - 1);
        it.next();
        const bool more = it.valid();
        // the workgroup's last tile overlaps with a copy of itself: its own
        // rows, and its last P k-steps again (just read, from L2)
        Tile nx = cur;
        if (more) setup(it.t, nx);
        const int nstep0 = more ? 0 : nsteps - P;
#pragma unroll
        for (int c = 0; c < kNB; ++c) accg[c] = accu[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < nsteps - P; s0 += P) {
#pragma unroll
            for (int p = 0; p < P; ++p) mma(p, s0 + p);
            refill(s0 + P, cur);
        }
#pragma unroll
        for (int p = 0; p < P; ++p) mma(p, nsteps - P + p);
        refill(nstep0, nx);

        // partial sums -> LDS; row = 4*(lane/16) + q, col = wave*32 + c*16 + lane%16
#pragma unroll
        for (int c = 0; c < kNB; ++c)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = wave * kNB * 16 + c * 16 + lane % 16;
                red[4 * kq + q][col] = accg[c][q];
                red[4 * kq + q][TN + col] = accu[c][q];
            }
        barrier_lds();   // also: every wave is past its last multiply
        load_rows(nx, 0, H);
        // SwiGLU, then MXFP8 along I (as in mx_gateup_kernel)
        constexpr int TQ = TN / 4;
        uint8_t* he = (uint8_t*)A.h_scale;
        const GroupInfo& gi = cur.gi;
        for (int e = tid; e < 16 * TQ; e += NT) {
            const int row = e / TQ, c4 = (e % TQ) * 4;
            float hv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float g = 0.f, u = 0.f;   // summed from zero as in mx_gateup_kernel (a -0 sum reads +0)
                g += red[row][c4 + j];
                u += red[row][TN + c4 + j];
                hv[j] = silu_mul(g, u);
            }
            float amax = fmaxf(fmaxf(fabsf(hv[0]), fabsf(hv[1])), fmaxf(fabsf(hv[2]), fabsf(hv[3])));
            amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
            amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
            amax = fmaxf(amax, __shfl_xor(amax, 4, kWave));
            const uint32_t E = mx_e8m0_for_e4m3(amax);
            const float f = mx_inv_scale(E);
            const uint32_t code = f32x4_to_e4m3x4(hv[0] * f, hv[1] * f, hv[2] * f, hv[3] * f);
            const int r = cur.m0 + row;
            if (r < gi.m) {
                const int hr = h_row(A, gi, r);
                *(uint32_t*)(A.h + (size_t)hr * I + cur.nt0 + c4) = code;
                if ((c4 & 31) == 0) he[(size_t)hr * (I / 32) + (cur.nt0 + c4) / 32] = (uint8_t)E;
            }
        }
        if (!more) {
            wait_vm<0>();   // no direct load into LDS outlives the workgroup
            break;
        }
        cur = nx;
        // this wave's rows of the new tile (and its first P k-steps) are in,
        // then everyone's; the barrier also orders the epilogue's reads of
        // `red` before the next tile's writes
        wait_vm<0>();
        barrier_lds();
    }
}

// ---------------------------------------------------------------- down
template <int MB, int P, int kNB, bool XEX, bool XP = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void mx_down_kernel(GArgs A, TileList L) {
    static_assert(!XP || (MB == 1 && kNB % 4 == 0 && P % 4 == 0 && !XEX), "packed exponents: weight blocks in fours");
    constexpr int TN = 4 * kNB * 16;           // output (H) columns per tile; each wave all of K
    constexpr int RS = TN + 1;
    const int H = A.H, I = A.I;
    const int ntn = H / TN;
    const int nsteps = I / 128;

    __shared__ float red[16 * MB][RS];

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int kq = lane / 16;
    const uint32_t esh = 8u * kq;
    const uint8_t* he = (const uint8_t*)A.h_scale;
    constexpr bool XE = XEX && P % 4 == 0 && 16 % P == 0;   // exponents in 16-step blocks

    for (TileIter it(L, ntn); it.valid(); it.next()) {
        const int t = (int)it.t;
        __syncthreads();
        const int2 tc = tile_coords<MB == 1>(L, t, ntn);
        const int2 tl = L.entries[tc.x];
        const GroupInfo gi = group_info(A, tl.x);
        const int m0 = tl.y;
        const int nt0 = tc.y * TN;
        const int n0 = nt0 + wave * kNB * 16;
        const Bank bk = gi.shared ? A.shared : A.routed;

        const uint8_t* ap[MB];
        const uint8_t* aep[MB];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            const int hr = h_row(A, gi, min(m0 + i * 16 + lane % 16, gi.m - 1));
            ap[i] = A.h + (size_t)hr * I + kq * 16;
            aep[i] = he + (size_t)hr * (I / 32);
        }
        const uint8_t *dp[kNB], *dep[kNB];
#pragma unroll
        for (int c = 0; c < kNB; ++c) {
            const size_t row = (size_t)gi.e * H + n0 + c * 16 + lane % 16;
            dp[c] = (const uint8_t*)bk.wd + row * (I / 2) + kq * 16;
            dep[c] = (const uint8_t*)bk.sd + row * (I / 32);
        }
        // XP: the packed exponents of the wave's weight blocks, 1 KiB per four
        // blocks (64 rows) and four steps
        const uint8_t* xpp = XP ? bk.xd + (((size_t)gi.e * (H / 64) + n0 / 64) * (I / 512)) * 1024 + lane * 16 : nullptr;
        i32x4 xpv[P / 4 > 0 ? P / 4 : 1][kNB / 4 > 0 ? kNB / 4 : 1];

        f32x4 acc[MB][kNB];
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int c = 0; c < kNB; ++c) acc[i][c] = f32x4{0.f, 0.f, 0.f, 0.f};

        i32x8 ra[P][MB];
        uint32_t rae[P][MB];
        i32x4 rd[P][kNB];
        uint32_t rde[P][kNB];
        i32x4 xcd[kNB], xca[MB], xnd[kNB], xna[MB];   // exponent blocks (XE): current, next
        auto load_w = [&](int p, int step) {
#pragma unroll
            for (int c = 0; c < kNB; ++c) rd[p][c] = gld<i32x4>(dp[c] + step * 64);
#pragma unroll
            for (int i = 0; i < MB; ++i) ra[p][i] = load_act(ap[i] + step * 128);
        };
        auto load_e = [&](int p, int step) {
            if constexpr (XP) {
                if ((p & 3) == 3)
#pragma unroll
                    for (int q = 0; q < kNB / 4; ++q)
                        xpv[p >> 2][q] = gld<i32x4>(xpp + ((size_t)q * (I / 512) + ((step - 3) >> 2)) * 1024);
            } else {
#pragma unroll
                for (int c = 0; c < kNB; ++c) rde[p][c] = gld<uint32_t>(dep[c] + step * 4);
            }
#pragma unroll
            for (int i = 0; i < MB; ++i) rae[p][i] = gld<uint32_t>(aep[i] + step * 4);
        };
        auto load_x = [&](int blk, i32x4 (&xd)[kNB], i32x4 (&xa)[MB]) {
#pragma unroll
            for (int c = 0; c < kNB; ++c) xd[c] = gld<i32x4>(dep[c] + blk * 64 + kq * 16);
#pragma unroll
            for (int i = 0; i < MB; ++i) xa[i] = gld<i32x4>(aep[i] + blk * 64 + kq * 16);
        };
        auto next_block = [&]() {
#pragma unroll
            for (int c = 0; c < kNB; ++c) xcd[c] = xnd[c];
#pragma unroll
            for (int i = 0; i < MB; ++i) xca[i] = xna[i];
        };
        auto mma = [&](int p, int s0, bool x) {
            uint32_t ea[MB], ed[kNB];
            if (x) {
                const int src = (lane & 15) + 16 * (((s0 + p) & 15) >> 2);
#pragma unroll
                for (int c = 0; c < kNB; ++c) ed[c] = xlane(src, xcd[c][p & 3]) >> esh;
#pragma unroll
                for (int i = 0; i < MB; ++i) ea[i] = xlane(src, xca[i][p & 3]) >> esh;
            } else if constexpr (XP) {
#pragma unroll
                for (int c = 0; c < kNB; ++c) ed[c] = (uint32_t)xpv[p >> 2][c >> 2][p & 3] >> (8 * (c & 3));
#pragma unroll
                for (int i = 0; i < MB; ++i) ea[i] = rae[p][i] >> esh;
            } else {
#pragma unroll
                for (int c = 0; c < kNB; ++c) ed[c] = rde[p][c] >> esh;
#pragma unroll
                for (int i = 0; i < MB; ++i) ea[i] = rae[p][i] >> esh;
            }
#pragma unroll
            for (int c = 0; c < kNB; ++c)
#pragma unroll
                for (int i = 0; i < MB; ++i) acc[i][c] = mma_f8f4(ra[p][i], rd[p][c], acc[i][c], ea[i], ed[c]);
        };
        const int nmain = XE ? nsteps / 16 * 16 : nsteps / P * P;
        if (XP && nmain > 0) {
            // the refill of the whole ring once its multiplies are issued:
            // the exponent records first, then each step's weights and
            // activations (with the records last, the compiler hoists their
            // shifts to the ring's first multiplies, which then wait for
            // every load)
            auto refill = [&](int step0) {
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int g = 0; g < P / 4; ++g)
#pragma unroll
                    for (int q = 0; q < kNB / 4; ++q)
                        xpv[g][q] = gld<i32x4>(xpp + ((size_t)q * (I / 512) + step0 / 4 + g) * 1024);
#pragma unroll
                for (int p = 0; p < P; ++p) {
                    load_w(p, step0 + p);
#pragma unroll
                    for (int i = 0; i < MB; ++i) rae[p][i] = gld<uint32_t>(aep[i] + (step0 + p) * 4);
                }
                __builtin_amdgcn_sched_barrier(0);
            };
            refill(0);
            int s0 = 0;
            for (; s0 < nmain - P; s0 += P) {
#pragma unroll
                for (int p = 0; p < P; ++p) mma(p, s0, false);
                refill(s0 + P);
            }
#pragma unroll
            for (int p = 0; p < P; ++p) mma(p, s0, false);
        } else if (nmain > 0) {
            if (XE) {
                load_x(0, xcd, xca);
                if (nmain > 16) load_x(1, xnd, xna);
            }
#pragma unroll
            for (int p = 0; p < P; ++p) {
                load_w(p, p);
                if (!XE) load_e(p, p);
            }
            int s0 = 0;
            for (; s0 < nmain - P; s0 += P) {
                if (XE && s0 > 0 && (s0 & 15) == 0) {
                    next_block();
                    if (s0 + 16 < nmain) load_x(s0 / 16 + 1, xnd, xna);
                }
#pragma unroll
                for (int p = 0; p < P; ++p) {
                    mma(p, s0, XE);
                    load_w(p, s0 + P + p);
                    if (!XE) load_e(p, s0 + P + p);
                }
            }
            if (XE && s0 > 0 && (s0 & 15) == 0) next_block();
#pragma unroll
            for (int p = 0; p < P; ++p) mma(p, s0, XE);
        }
        for (int s = nmain; s < nsteps; ++s) {
            load_w(0, s);
            load_e(0, s);
            mma(0, s, false);
        }

#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int c = 0; c < kNB; ++c)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    red[i * 16 + 4 * (lane / 16) + q][wave * kNB * 16 + c * 16 + lane % 16] = acc[i][c][q];
        __syncthreads();
        void* yb = gi.shared ? A.y_sh : A.y;
        const int ybf = gi.shared ? A.y_sh_bf16 : A.y_bf16;
        for (int e = tid; e < 16 * MB * TN; e += 256) {
            const int row = e / TN, col = e % TN;
            const int r = m0 + row;
            if (r >= gi.m) continue;
            const float v = red[row][col];
            const size_t yr = gi.shared ? (size_t)r : (size_t)(gi.p0 + r);
            if (ybf) ((uint16_t*)yb)[yr * H + nt0 + col] = (uint16_t)f32_to_bf16_bits(v);
            else ((float*)yb)[yr * H + nt0 + col] = v;
        }
    }
}

// ---------------------------------------------------------------- launchers
template <class K>
static int mx_persistent_grid(K kernel) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) != hipSuccess || per_cu < 1) per_cu = 1;
    return per_cu * device_cu_count();
}

#define MOE_MX_LAUNCH(KERNEL)                                                       \
    do {                                                                            \
        static DeviceCache cache_;                                                  \
        const int g = per_device(cache_, [] { return mx_persistent_grid(KERNEL); }); \
        hipLaunchKernelGGL(KERNEL, dim3(g), dim3(256), 0, s, A, L);                 \
    } while (0)

// The K split of gate/up over two waves needs an even number of 128-wide
// k-steps (H % 256 == 0); otherwise every wave covers all of K.  Tiles of 16
// rows keep 4 k-steps of loads in flight, tiles of 64 rows 2 (registers).
// Tuning of the 16-row MX tiles (measured on the T = 128 decode layer):
// gate/up covers all of K per wave (no split) with 8 k-steps in flight, two
// 16-column blocks per wave and an exponent dword per step; down keeps 4
// k-steps in flight over four 16-column blocks with 16-step exponent blocks.
constexpr int kMxGuKs = 1, kMxGuP = 8, kMxGuNb = 2;
constexpr bool kMxGuXe = false;
constexpr int kMxDnP = 4, kMxDnNb = 4;
// down with packed exponents: eight 16-column blocks per wave (512-column
// tiles), which doubles the weight bytes in flight per wave and halves the
// tiles a decode layer starts
constexpr int kMxDnNbXp = 8;
// 16-row gate/up tiles stage the tile's activation rows and exponents in LDS
// where they fit beside the 16 KiB partial-sum table (H up to 8192): decode
// layer T = 128 gate/up 0.77 -> 0.74 ms.  Exponent dwords per step there: the
// 16-step exponent blocks were slower (0.85 ms).
constexpr size_t kMxGuLdsMax = 140 * 1024;
// waves of the overlapped 16-row gate/up workgroup (one per CU: LDS): eight
// waves share one copy of the tile's activation rows over 256 h columns and
// keep twice the weight bytes in flight
constexpr int kMxGuOvlWaves = 8;
constexpr bool kMxDnXe = true;
// 16-row tiles.  gate/up: K split over kMxGuKs waves when the 128-wide
// k-steps divide evenly, kMxGuNb column blocks per wave when I is a
// multiple of the tile width (else 2), 8 k-steps in flight with an exponent
// dword per step (the 16-step exponent blocks need registers that a ring of
// 8 leaves no room for, and a ring of 4 with them measured 1% slower).
// down: 4 k-steps in flight with 16-step exponent blocks (5% faster than
// per-step exponents).  64-row tiles: two k-steps in flight (registers).
hipError_t launch_mx_gateup(int mb, const GArgs& A, const TileList& L, hipStream_t s) {
    const int nst = A.H / 128;
    constexpr int KS = kMxGuKs, NB = kMxGuNb;
    constexpr bool XE = kMxGuXe;
    static_assert(KS == 1 || KS == 2 || KS == 4, "K split over 1, 2 or 4 waves");
    const size_t alds = (size_t)16 * (A.H + 16) + (size_t)16 * (A.H / 32 + 4);
    if (mb == 1 && alds <= kMxGuLdsMax && A.I % (4 * NB * 16) == 0) {
        // packed exponents: both banks carry them, and the ring covers K
        // exactly; consecutive tiles overlapped where K has at least two rings
        const bool xp = A.routed.xgu && (A.S == 0 || A.shared.xgu) && A.H % 1024 == 0;
        // the overlapped kernel's partial-sum table (static LDS) beside the rows
        constexpr size_t kOvlRed = (size_t)16 * (2 * kMxGuOvlWaves * NB * 16 + 1) * sizeof(float);
        constexpr size_t kOvlLdsMax = (size_t)160 * 1024 - kOvlRed;
        const bool ovl = xp && nst >= 2 * kMxGuP && A.I % (kMxGuOvlWaves * NB * 16) == 0 && alds <= kOvlLdsMax;
        static_assert(NB == 2 && 1024 % (128 * kMxGuP) == 0, "overlapped tiles: two blocks per wave, H / 128 a multiple of P");
        auto k = ovl ? mx_gateup_ovl_kernel<kMxGuP, kMxGuOvlWaves>
               : xp  ? mx_gateup_kernel<1, 1, kMxGuP, NB, false, true, true>
                     : mx_gateup_kernel<1, 1, kMxGuP, NB, false, true>;
        static DeviceCache cache, cache_xp, cache_ovl;
        const int g = per_device(ovl ? cache_ovl : xp ? cache_xp : cache, [k, ovl] {
            (void)hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                      (int)(ovl ? kOvlLdsMax : kMxGuLdsMax));
            return device_cu_count();   // one workgroup per CU (LDS)
        });
        hipLaunchKernelGGL(k, dim3(g), dim3(ovl ? 64 * kMxGuOvlWaves : 256), alds, s, A, L);
        return hipGetLastError();
    }
    if (mb == 1) {
        if (nst % KS == 0 && A.I % (4 / KS * NB * 16) == 0) MOE_MX_LAUNCH((mx_gateup_kernel<1, KS, kMxGuP, NB, XE>));
        else MOE_MX_LAUNCH((mx_gateup_kernel<1, 1, kMxGuP, 2, XE>));
    } else {
        if (nst % 2 == 0) MOE_MX_LAUNCH((mx_gateup_kernel<4, 2, 2, 2, false>));
        else MOE_MX_LAUNCH((mx_gateup_kernel<4, 1, 2, 2, false>));
    }
    return hipGetLastError();
}

hipError_t launch_mx_down(int mb, const GArgs& A, const TileList& L, hipStream_t s) {
    constexpr int NB = kMxDnNb;
    constexpr bool XE = kMxDnXe;
    // packed exponents (banks packed only with H % 1024 == 0 and I % 512 == 0)
    if (mb == 1 && A.routed.xd && (A.S == 0 || A.shared.xd) && A.H % (64 * kMxDnNbXp) == 0 && A.I % 512 == 0) {
        MOE_MX_LAUNCH((mx_down_kernel<1, kMxDnP, kMxDnNbXp, false, true>));
        return hipGetLastError();
    }
    if (mb == 1) {
        if (A.H % (64 * NB) == 0) MOE_MX_LAUNCH((mx_down_kernel<1, kMxDnP, NB, XE>));
        else MOE_MX_LAUNCH((mx_down_kernel<1, kMxDnP, 2, XE>));
    } else {
        MOE_MX_LAUNCH((mx_down_kernel<4, 2, 2, false>));
    }
    return hipGetLastError();
}
#undef MOE_MX_LAUNCH

// ---------------------------------------------------------------- packed exponents
// One thread per 16-byte lane record of the packed layouts (include/moe.h,
// moe_mx_pack_scales): record (e, blk, j, lane), byte q = 4 ss + b.
__global__ __launch_bounds__(256) void mx_pack_gu_kernel(int n, int H, int I, const uint8_t* __restrict__ sg,
                                                         const uint8_t* __restrict__ su, uint8_t* __restrict__ out) {
    const int nj = H / 512, nb = I / 32, KB = H / 32;
    const long rec = (long)blockIdx.x * 256 + threadIdx.x;
    if (rec >= (long)n * nb * nj * 64) return;
    const int lane = (int)(rec % 64);
    const long t = rec / 64;
    const int j = (int)(t % nj), blk = (int)(t / nj % nb), e = (int)(t / nj / nb);
    const int c = lane / 16, r = lane % 16;
    uint8_t v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int ss = q / 4, b = q % 4;
        const uint8_t* src = b < 2 ? sg : su;
        v[q] = src[((size_t)e * I + 32 * blk + 16 * (b & 1) + r) * KB + 4 * (4 * j + ss) + c];
    }
    *(i32x4*)(out + rec * 16) = *(const i32x4*)v;
}

__global__ __launch_bounds__(256) void mx_pack_d_kernel(int n, int H, int I, const uint8_t* __restrict__ sd,
                                                        uint8_t* __restrict__ out) {
    const int nj = I / 512, nb = H / 64, KB = I / 32;
    const long rec = (long)blockIdx.x * 256 + threadIdx.x;
    if (rec >= (long)n * nb * nj * 64) return;
    const int lane = (int)(rec % 64);
    const long t = rec / 64;
    const int j = (int)(t % nj), blk = (int)(t / nj % nb), e = (int)(t / nj / nb);
    const int c = lane / 16, r = lane % 16;
    uint8_t v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int ss = q / 4, b = q % 4;
        v[q] = sd[((size_t)e * H + 64 * blk + 16 * b + r) * KB + 4 * (4 * j + ss) + c];
    }
    *(i32x4*)(out + rec * 16) = *(const i32x4*)v;
}

hipError_t launch_mx_pack_scales(int n, int H, int I, const uint8_t* sg, const uint8_t* su, const uint8_t* sd,
                                 uint8_t* xgu, uint8_t* xd, hipStream_t s) {
    if (xgu) {
        const long recs = (long)n * (I / 32) * (H / 512) * 64;
        hipLaunchKernelGGL(mx_pack_gu_kernel, dim3((unsigned)((recs + 255) / 256)), dim3(256), 0, s, n, H, I, sg, su, xgu);
    }
    if (xd) {
        const long recs = (long)n * (H / 64) * (I / 512) * 64;
        hipLaunchKernelGGL(mx_pack_d_kernel, dim3((unsigned)((recs + 255) / 256)), dim3(256), 0, s, n, H, I, sd, xd);
    }
    return hipGetLastError();
}

}  // namespace moe
