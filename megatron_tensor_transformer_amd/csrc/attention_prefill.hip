// Causal grouped-query attention for a block of new tokens (prefill).
//
// The S tokens of a sequence sit at positions kv_len - S .. kv_len - 1 and
// their k, v are already in the cache; the token at position p attends to
// positions 0..p with scores scaled by 1/sqrt(D), and query head h reads kv
// head h / GQ.
//
// Work split. A query block is 64 rows: 64 / GQ consecutive tokens x the GQ
// heads of one kv head, so every K and V block staged for it serves all of
// them. Causality makes late query blocks see many more keys than early
// ones, so a workgroup takes two query blocks of one (sequence, kv head),
// i and n - 1 - i, one after the other: every workgroup then walks about the
// same number of keys and the grid ends together. Inside a query block the 8
// waves split the work 2 x 4: wave w owns rows 32 (w % 2) .. + 31 (two MFMA
// column tiles of 16) and keys 32 (w / 2) .. + 31 of every 128-key block,
// with its own running softmax state; the four key quarters of a row are
// merged by their log-sum-exp weights through LDS at the end.
//  - Scores are computed transposed, S^T = K Q^T, on
//    v_mfma_f32_16x16x32_bf16: a lane then holds one query row's scores for
//    four keys of each 16-key tile, so the softmax of a row needs only its
//    own lane and the three lanes that share its column (two permlane swaps),
//    and the probabilities already form the B operand of O^T = V^T P^T
//    (a lane's 8 k-values are keys 4kg..4kg+3 of the wave's two key tiles;
//    the V^T operand reads the same 8 keys).
//  - K and V go through LDS in blocks of 128 keys, double buffered, one
//    barrier per block: once a block's LDS reads are issued, the next
//    block's K and V go straight from global memory into the other stage
//    (buffer loads to LDS), both as rows of D elements with their 16-byte
//    chunks XOR-swizzled by key. V^T operands come out of the V rows with
//    LDS transpose reads (ds_read_b64_tr_b16): in each group of 16 lanes,
//    lane i receives element i % 4 of the 8 bytes that lanes 4j + i / 4
//    point at, j = 0..3, so lanes pointing at 4 keys x 4 consecutive d
//    quarters deliver V[key j][d] for lane d: the 4 keys of a lane's
//    probabilities in one 16-key tile. Each wave reads its K fragments of a
//    block at once, ahead of the score products, and its V fragments behind
//    them, ahead of the softmax.
//  - The online softmax (running max and sum per row, in the base-2 domain
//    with the 1/sqrt(D) scale folded into one multiply-add) runs in
//    registers. The reference maximum is raised only when a score exceeds it
//    by more than 2^PF_SLACK, so most blocks skip the rescale of the
//    accumulators. Probabilities are rounded to bf16 and the running sum
//    adds exactly the rounded values (one v_dot2 with (1, 1) per key pair).
//  - Causality: a query block walks key blocks up to its last token's
//    position; only blocks that reach past its first token's position are
//    masked, and a wave skips a quarter that lies wholly past every row.
#include "device_common.h"
#include "kernels.h"

namespace tpk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int PF_NT = 512;       // threads (8 waves)
constexpr int PF_ROWS = 64;      // query rows per query block
constexpr int PF_BK = 128;       // keys per block
constexpr int PF_KW = 32;        // keys per wave per block
constexpr float PF_SLACK = 8.0f; // log2 of the largest unnormalised probability
constexpr float PF_LOG2E = 1.4426950408889634f;

__device__ __forceinline__ f32x4_t mfma16x32(const uint4& a, const uint4& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

// Maxima of finite or -inf scores: the IEEE maximum, which needs no quieting
// of NaN operands first (fmaxf costs an extra instruction per operand) and
// becomes v_maximum3_f32 on gfx950. A compiler operation, not inline asm, so
// that the compiler keeps the wait states a matrix instruction's result needs
// before a vector instruction reads it.
__device__ __forceinline__ float pf_max3(float a, float b, float c) {
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}
__device__ __forceinline__ float pf_max2(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// op over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lanes of one MFMA
// column): between the two results of a swap with itself every lane holds its
// own value and its partner's, so op(a, b) needs no lane selects.
__device__ __forceinline__ float pf_max4(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = pf_max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
    auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return pf_max2(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float pf_sum4(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// Position of V chunk lc (16 bytes) of key row r in the V tile: XOR with an
// even value from the key, so that the 8 keys x 2 chunks the 32 lanes of one
// transpose read touch fall into 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int v_chunk(int r, int lc) {
    return lc ^ (D == 128 ? ((r & 7) << 1) : (((r >> 1) & 3) << 1));
}

// Position of K chunk lc (16 bytes) of key row r in the unpadded K tile: the
// chunk index is XOR-swizzled with bits of the row, so that the 16 rows a
// quarter-wave reads for one MFMA operand fall into distinct LDS banks.
template <int D>
__device__ __forceinline__ int k_chunk(int r, int lc) {
    return lc ^ (D == 128 ? (r & 15) : ((r >> 1) & 7));
}

// Buffer view of one key block of a head's K or V rows: the block's first
// row as base and its rows below kv_len as the range. Reads past the range
// return zeros, so keys past kv_len need no clamping (their scores are
// masked), and the per-lane offsets stay the same from block to block.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t key_block(const uint16_t* rows, int key0, int nvalid, int d) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(rows + (size_t)key0 * d), (short)0,
                                             min(nvalid, PF_BK) * d * 2, 0x00020000);
}
// The transfer of 16 bytes per lane from the buffer at byte offset off into
// LDS at lds_base + 16 lane. Written out rather than through the builtin:
// the compiler orders every later LDS read behind a transfer into LDS it
// knows of (it cannot tell that they read the other stage), which would keep
// the next block's transfers from being issued ahead of this block's reads.
// The kernel waits for them itself (s_waitcnt vmcnt(0) before the barrier
// that hands the stage over). The compiler writes M0 right before the
// block; an LDS transfer needs one wait state after an M0 write (the
// compiler puts the same s_nop before its own), which it cannot see here.
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, unsigned off, uint16_t* lds_base) {
    const unsigned lds = (unsigned)(uintptr_t)(__attribute__((address_space(3))) void*)lds_base;
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(r), "{m0}"(lds) : "memory");
}
typedef short pf_s4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
    const pf_s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) pf_s4*)p);
    return __builtin_bit_cast(uint2, v);
}

template <int D, int GQ>
__global__ __launch_bounds__(PF_NT, 1) void attn_prefill_kernel(PrefillArgs a) {
    constexpr int KDMA = PF_BK * D * 2 / 1024 / 8; // 1 KB transfers per wave per K (or V) block
    constexpr int DS = D / 32;                     // MFMA steps over d for the scores
    constexpr int DT = D / 16;                     // 16-wide d tiles of the output
    constexpr int TOK = PF_ROWS / GQ;              // tokens per query block
    constexpr int KTILE = PF_BK * D;               // elements
    constexpr int VTILE = PF_BK * D;
    constexpr int NV = DT * 8 + 4;                 // floats a lane publishes in the merge (NV / 4 float4)
    static_assert(KDMA >= 1, "blocks must split evenly over the threads");

    // Two stages, each a K tile then a V tile. The merge areas (four of NV
    // floats per lane) start at the second stage, clear of the first, which
    // meanwhile takes the next query block's first K and V block.
    constexpr int BUF = KTILE + VTILE;
    constexpr int MERGE_END = BUF + 4 * NV * 64 * 2;  // elements
    __shared__ __align__(16) uint16_t smem[2 * BUF > MERGE_END ? 2 * BUF : MERGE_END];
    static_assert(sizeof(smem) <= 160 * 1024, "LDS of one compute unit");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS bases stay scalar
    const int rg = wave & 1, kq = wave >> 1;      // row group, key quarter
    const int col = lane & 15, kg = lane >> 4;
    const int heads = a.kv_heads * a.batch;
    const int pair = (int)(blockIdx.x / heads);
    const int g = (int)(blockIdx.x % heads) % a.kv_heads, b = (int)(blockIdx.x % heads) / a.kv_heads;
    const int S = a.seq, kv_len = a.kv_len;
    const int p0 = kv_len - S;                      // position of token 0 of the block
    const int nqb = (S + TOK - 1) / TOK;

    const size_t head_off = ((size_t)b * a.kv_heads + g) * a.capacity * D;
    const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.k) + head_off;
    const uint16_t* vbase = reinterpret_cast<const uint16_t*>(a.v) + head_off;
    const uint16_t* qbase = reinterpret_cast<const uint16_t*>(a.q);
    uint16_t* obase = reinterpret_cast<uint16_t*>(a.out);
    const float c = PF_LOG2E / sqrtf((float)D);     // scores to the base-2 domain

    // K block: wave transfer i covers tile bytes [(i * 8 + wave) KB, + 1 KB),
    // lane L the 16 bytes at L * 16 in it: row e / D, physical chunk
    // (e % D) / 8, which holds logical chunk k_chunk(row, physical).
    unsigned koff[KDMA];                            // byte offsets within a key block
#pragma unroll
    for (int i = 0; i < KDMA; ++i) {
        const int e = (i * 8 + wave) * 512 + lane * 8;
        const int r = e / D;
        koff[i] = (unsigned)(r * D + k_chunk<D>(r, (e % D) / 8) * 8) * 2u;
    }
    auto load_k = [&](int kb, uint16_t* kdst) {
        const int key0 = kb * PF_BK;
        const __amdgpu_buffer_rsrc_t r = key_block(kbase, key0, kv_len - key0, D);
#pragma unroll
        for (int i = 0; i < KDMA; ++i) dma16_buf(r, koff[i], kdst + (i * 8 + wave) * 512);
    };
    // V block: as K, row e / D of the tile from transfer i, chunk swizzled by
    // v_chunk.
    unsigned voff[KDMA];
#pragma unroll
    for (int i = 0; i < KDMA; ++i) {
        const int e = (i * 8 + wave) * 512 + lane * 8;
        const int r = e / D;
        voff[i] = (unsigned)(r * D + v_chunk<D>(r, (e % D) / 8) * 8) * 2u;
    }
    auto load_v = [&](int kb, uint16_t* vdst) {
        const int key0 = kb * PF_BK;
        const __amdgpu_buffer_rsrc_t r = key_block(vbase, key0, kv_len - key0, D);
#pragma unroll
        for (int i = 0; i < KDMA; ++i) dma16_buf(r, voff[i], vdst + (i * 8 + wave) * 512);
    };
    // Transpose reads of a lane (group kg = lane / 16, r = lane % 16): key
    // 32 kq + 4 kg + r / 4 (+ 16 for the second), d quarter 4 (r % 4) of
    // each 16-wide d tile.
    const int tr_key = kq * PF_KW + kg * 4 + ((lane & 15) >> 2);
    const int tr_q = lane & 3;
    // The lane's fragment offsets within a tile (elements), the same for
    // every block: K rows 32 kq + col, chunk s * 4 + kg; V^T of d tile dt.
    // The second 16 rows (keys) of either are 16 D further on, since both
    // swizzles repeat every 16 rows.
    int kfo[DS], vto[DT];
#pragma unroll
    for (int s = 0; s < DS; ++s) {
        const int r = kq * PF_KW + col;
        kfo[s] = r * D + k_chunk<D>(r, s * 4 + kg) * 8;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        const int cc = dt * 2 + (tr_q >> 1);
        vto[dt] = tr_key * D + v_chunk<D>(tr_key, cc) * 8 + (tr_q & 1) * 4;
    }
    // The query fragments of this lane's two rows of query block qb (one row
    // per MFMA column tile): token qb TOK + r / GQ, head g GQ + r % GQ.
    uint4 qf[2][DS];
    auto load_q = [&](int qb) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int r = rg * 32 + rt * 16 + col;
            const int tk = min(qb * TOK + r / GQ, S - 1);
            const int hq = g * GQ + r % GQ;
            const uint16_t* qrow = qbase + ((size_t)b * S + tk) * a.q_stride + (size_t)hq * D;
#pragma unroll
            for (int s = 0; s < DS; ++s) qf[rt][s] = load_u4(qrow + s * 32 + kg * 8);
        }
    };
    // Query blocks pair and nqb - 1 - pair (once when they coincide). The
    // first walks its key blocks backwards and so ends on block 0 (in stage
    // 0), which the second walks first, forwards: only the second block's
    // query fragments are requested between them, during the first one's
    // merge, which works above stage 0. Block kb always sits in stage kb % 2.
    int qblk = pair;
    {
        const int nblk0 = (p0 + min(qblk * TOK + TOK, S) - 1) / PF_BK + 1;
        load_q(qblk);
        load_k(nblk0 - 1, smem + ((nblk0 - 1) & 1) * BUF);
        load_v(nblk0 - 1, smem + ((nblk0 - 1) & 1) * BUF + KTILE);
    }
    for (int ph = 0; ph < 2; ++ph) {
        const int i0 = qblk * TOK;                  // first token of the query block
        const int ilast = min(i0 + TOK, S) - 1;
        const int nblk = (p0 + ilast) / PF_BK + 1;  // blocks up to the last token's position
        const int nfull = (p0 + i0 + 1) / PF_BK;    // blocks every row sees whole
        const int plast = p0 + ilast;

        // This lane's two query rows: token and position.
        int tok[2], pos[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            tok[rt] = i0 + (rg * 32 + rt * 16 + col) / GQ;
            pos[rt] = p0 + tok[rt];
        }

        float mrun[2] = {-INFINITY, -INFINITY}, lrun[2] = {0.f, 0.f};
        // Row sums of the rounded probabilities. With d = 128 on the matrix
        // cores: an all-ones A operand times P^T gives every row's sum in
        // each of the lane's four outputs, accumulated and rescaled like the
        // outputs (fewer vector instructions; the 8 registers it takes would
        // cost d = 64 a workgroup per compute unit, so there the lanes add
        // their probabilities with v_dot2 and two permlane swaps).
        constexpr bool MSUM = D == 128;
        f32x4_t lacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
        const uint4 ones = make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u);
        f32x4_t ot[DT][2];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) ot[dt][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        // Every load issued so far (the query fragments included) has landed,
        // so the waits inside the loop only ever cover the next block's loads;
        // past this barrier every wave has also left the last merge.
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();

        // One block for this wave, its 32 keys x its 32 rows, in two halves:
        // the front reads every LDS fragment it needs and forms the scores, the
        // back weighs them and accumulates the outputs.
        f32x4_t st[2][2];
        uint4 vf[DT];
        auto front = [&](const uint16_t* kt, const uint16_t* vtb) {
            // The block's K fragments first, all at once.
            uint4 kf[DS][2];
#pragma unroll
            for (int s = 0; s < DS; ++s)
#pragma unroll
                for (int t = 0; t < 2; ++t) kf[s][t] = *reinterpret_cast<const uint4*>(&kt[kfo[s] + t * 16 * D]);
            __builtin_amdgcn_sched_barrier(0);

            // S^T tiles: keys 32 kq + 16 t .. + 15 of the block x this wave's
            // rows; four independent accumulation chains.
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) st[t][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < DS; ++s)
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt) st[t][rt] = mfma16x32(kf[s][t], qf[rt][s], st[t][rt]);

            // V^T fragments (the same 8 keys per lane as the probabilities),
            // read now so that they land during the softmax.
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const uint2 lo = lds_read_tr16(&vtb[vto[dt]]);
                const uint2 hi = lds_read_tr16(&vtb[vto[dt] + 16 * D]);
                vf[dt] = make_uint4(lo.x, lo.y, hi.x, hi.y);
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        auto back = [&](int kb, bool masked) {
            // Online softmax; the lane holds keys 32 kq + 16 t + 4 kg + j.
            float mx[2];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                if (masked) {
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int key = kb * PF_BK + kq * PF_KW + t * 16 + kg * 4 + j;
                            if (key > pos[rt]) st[t][rt][j] = -INFINITY;
                        }
                }
                const float m8 = pf_max3(pf_max3(st[0][rt][0], st[0][rt][1], st[0][rt][2]),
                                         pf_max3(st[0][rt][3], st[1][rt][0], st[1][rt][1]),
                                         pf_max2(st[1][rt][2], st[1][rt][3]));
                mx[rt] = pf_max4(m8) * c;
            }
            const bool grow = mx[0] > mrun[0] + PF_SLACK || mx[1] > mrun[1] + PF_SLACK;
            if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    const float mnew = fmaxf(mrun[rt], mx[rt]);
                    const float al = __builtin_amdgcn_exp2f(mrun[rt] - (mnew == -INFINITY ? 0.f : mnew));
                    mrun[rt] = mnew;
                    if (MSUM) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) lacc[rt][j] *= al;
                    } else {
                        lrun[rt] *= al;
                    }
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                        for (int j = 0; j < 4; ++j) ot[dt][rt][j] *= al;
                }
            }
            uint4 pk[2];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const float mref = mrun[rt] == -INFINITY ? 0.f : mrun[rt];
                float sum = 0.f;
                uint32_t pw[2][2];
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[t][rt][2 * h2], c, -mref));
                        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[t][rt][2 * h2 + 1], c, -mref));
                        pw[t][h2] = pack_bf16x2(e0, e1);
                        if (!MSUM) sum = dot2_bf16(pw[t][h2], 0x3f803f80u, sum);
                    }
                if (!MSUM) lrun[rt] += pf_sum4(sum);
                pk[rt] = make_uint4(pw[0][0], pw[0][1], pw[1][0], pw[1][1]);
            }
            __builtin_amdgcn_sched_barrier(0);

            // O^T += V^T P^T, and the row sums.
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) ot[dt][rt] = mfma16x32(vf[dt], pk[rt], ot[dt][rt]);
            if (MSUM) {
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) lacc[rt] = mfma16x32(ones, pk[rt], lacc[rt]);
            }
        };

        // One block for the workgroup; kn is the block that follows it (-1:
        // none). The next block's K and V go by DMA into the other stage
        // first thing, so that they have the whole block to land: every read
        // of that stage ended before the last barrier.
        auto step = [&](int kb, int kn, bool masked) {
            const int buf = kb & 1;
            const bool more = kn >= 0;
            uint16_t* cur = smem + buf * BUF;
            uint16_t* nxt = smem + (buf ^ 1) * BUF;
            if (more) {
                load_k(kn, nxt);
                load_v(kn, nxt + KTILE);
            }
            // a quarter wholly past the last token's position holds no visible key
            const bool active = !masked || kb * PF_BK + kq * PF_KW <= plast;
            if (active) front(cur, cur + KTILE);
            if (active) back(kb, masked);
            if (more) __builtin_amdgcn_s_waitcnt(0);  // the K and V transfers have landed in LDS
            __syncthreads();
        };
        // Blocks every row sees whole and the diagonal ones in loops of their
        // own, so that each has a single body: the first query block from its
        // last block down to block 0, the second from block 0 up.
        if (ph == 0) {
            int kb = nblk - 1;
            for (; kb >= nfull; --kb) step(kb, kb - 1, true);
            for (; kb >= 0; --kb) step(kb, kb - 1, false);
        } else {
            int kb = 0;
            for (; kb < nfull; ++kb) step(kb, kb + 1 < nblk ? kb + 1 : -1, false);
            for (; kb < nblk; ++kb) step(kb, kb + 1 < nblk ? kb + 1 : -1, true);
        }
        if (MSUM) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) lrun[rt] = lacc[rt][0];
        }

        // The next query block's fragments, under this block's merge; its
        // first K and V block is block 0, still in stage 0.
        const int qnext = nqb - 1 - pair;
        const bool next = ph == 0 && qnext != pair;
        if (next) load_q(qnext);

        // Merge the key quarters by their log-sum-exp weights, in two rounds:
        // quarters 2, 3 into 0, 1, then 1 into 0. Layout [float4][lane]:
        // (m, l) of both rows first, then the outputs by (d tile, row tile).
        auto publish = [&](float* mg) {
            float4* m4 = reinterpret_cast<float4*>(mg);
            m4[lane] = make_float4(mrun[0], lrun[0], mrun[1], lrun[1]);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
                    m4[(1 + dt * 2 + rt) * 64 + lane] =
                        make_float4(ot[dt][rt][0], ot[dt][rt][1], ot[dt][rt][2], ot[dt][rt][3]);
        };
        auto combine = [&](const float* mg) {
            const float4* m4 = reinterpret_cast<const float4*>(mg);
            const float4 ml = m4[lane];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const float mb = rt ? ml.z : ml.x, lb = rt ? ml.w : ml.y;
                const float m = fmaxf(mrun[rt], mb);
                const float mr = m == -INFINITY ? 0.f : m;      // both halves empty: stay empty
                const float wa = __builtin_amdgcn_exp2f(mrun[rt] - mr), wb = __builtin_amdgcn_exp2f(mb - mr);
                mrun[rt] = m;
                lrun[rt] = lrun[rt] * wa + lb * wb;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const float4 o = m4[(1 + dt * 2 + rt) * 64 + lane];
                    ot[dt][rt][0] = ot[dt][rt][0] * wa + o.x * wb;
                    ot[dt][rt][1] = ot[dt][rt][1] * wa + o.y * wb;
                    ot[dt][rt][2] = ot[dt][rt][2] * wa + o.z * wb;
                    ot[dt][rt][3] = ot[dt][rt][3] * wa + o.w * wb;
                }
            }
        };
        auto region = [&](int i) -> float* { return reinterpret_cast<float*>(smem + BUF) + i * NV * 64; };
        if (kq >= 2) publish(region(rg * 2 + (kq - 2)));
        __syncthreads();
        if (kq < 2) combine(region(rg * 2 + kq));
        __syncthreads();
        if (kq == 1) publish(region(rg));
        __syncthreads();
        if (kq == 0) {
            combine(region(rg));
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                if (tok[rt] >= S) continue;
                const float inv = 1.0f / lrun[rt];
                const int r = rg * 32 + rt * 16 + col;
                const int hq = g * GQ + r % GQ;
                uint16_t* orow = obase + (((size_t)b * S + tok[rt]) * a.q_heads + hq) * D;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    *reinterpret_cast<uint2*>(orow + dt * 16 + kg * 4) =
                        make_uint2(pack_bf16x2(ot[dt][rt][0] * inv, ot[dt][rt][1] * inv),
                                   pack_bf16x2(ot[dt][rt][2] * inv, ot[dt][rt][3] * inv));
            }
        }
        if (!next) break;
        qblk = qnext;
    }
}

template <int D>
static hipError_t prefill_launch_d(const PrefillArgs& a, int gq, hipStream_t s) {
    const int tok = PF_ROWS / gq;
    const int64_t nqb = (a.seq + tok - 1) / tok;
    const int64_t blocks = (nqb + 1) / 2 * a.kv_heads * a.batch;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    dim3 grid((unsigned)blocks);
    switch (gq) {
        case 1: hipLaunchKernelGGL((attn_prefill_kernel<D, 1>), grid, dim3(PF_NT), 0, s, a); break;
        case 2: hipLaunchKernelGGL((attn_prefill_kernel<D, 2>), grid, dim3(PF_NT), 0, s, a); break;
        case 4: hipLaunchKernelGGL((attn_prefill_kernel<D, 4>), grid, dim3(PF_NT), 0, s, a); break;
        case 8: hipLaunchKernelGGL((attn_prefill_kernel<D, 8>), grid, dim3(PF_NT), 0, s, a); break;
        case 16: hipLaunchKernelGGL((attn_prefill_kernel<D, 16>), grid, dim3(PF_NT), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t prefill_attn_launch(const PrefillArgs& a, hipStream_t s) {
    const int gq = a.q_heads / a.kv_heads;
    if (a.head_dim == 64) return prefill_launch_d<64>(a, gq, s);
    if (a.head_dim == 128) return prefill_launch_d<128>(a, gq, s);
    return hipErrorInvalidValue;
}

}  // namespace tpk
