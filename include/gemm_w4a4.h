/*
 * gemm_w4a4.h — C ABI of the fused NVFP4 W4A4 GEMM for AMD Instinct MI355X (gfx950).
 *
 * The operation (section 2 of the SVDQuant W4A4 on Blackwell page,
 * "Blackwell 上的 SVDQuant W4A4 算子实现"):
 *
 *     y[m,n] = wcscale[n] * sum_k A[m,k] * W[n,k] + bias[n]
 *              + sum_r lora_act_in[m,r] * lora_up[r,n]
 *
 * where A and W are NVFP4: E2M1 codes (two per byte) times one FP8-E4M3 block
 * scale per 16 consecutive k (same page, section 3.1: single-level block
 * scaling, no per-tensor factor). The per-column affine is the page's
 * section 6.6 epilogue; the LoRA residual is added after the wcscale product,
 * as the section 2 formula writes it. The result is rounded to bfloat16
 * (nearest, ties to even).
 *
 * Layouts: every tensor is dense and row-major, without padding or strides.
 *   act          uint8   [M, K/2]   byte j of row m holds k = 2j (low nibble)
 *                                   and k = 2j+1 (high nibble)
 *   ascales      uint8   [K/16, M]  OCP E4M3FN bytes; scale of (m,k) is
 *                                   ascales[k/16][m]
 *   wgt          uint8   [N, K/2]   as act, one row per output column n
 *   wscales      uint8   [K/16, N]
 *   wcscale      float   [N]
 *   bias         float   [N]
 *   lora_act_in  uint16  [M, R]     bfloat16 bit patterns
 *   lora_up      uint16  [R, N]     bfloat16 bit patterns
 *   out          uint16  [M, N]     bfloat16 bit patterns (written)
 *
 * Ownership: every tensor pointer is a device pointer owned by the caller.
 * The library allocates and frees nothing, keeps no per-call state, and never
 * synchronizes: a successful call only enqueues work on `stream`.
 */
#ifndef GEMM_W4A4_H
#define GEMM_W4A4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. Validation runs before any HIP call, so on a negative code
 * nothing has been enqueued. No C++ exception crosses this boundary. */
enum {
  GEMM_W4A4_OK = 0,
  GEMM_W4A4_EINVAL = -1,      /* bad size (M<1, N<1, K<16, K%16, R<0, R>GEMM_W4A4_MAX_R,
                                 or any tensor of 2^31 bytes or more) or a required
                                 NULL pointer */
  GEMM_W4A4_EALIGN = -2,      /* act/wgt not 16-byte aligned, wcscale/bias not 4-byte,
                                 lora/out not 2-byte aligned */
  GEMM_W4A4_ELAUNCH = -3,     /* the HIP launch itself failed */
  GEMM_W4A4_EOVERLAP = -4,    /* out overlaps an input */
  GEMM_W4A4_EDEVICE = -5,     /* the current device is not gfx950 */
  GEMM_W4A4_ENOMEM = -6,      /* quantize_w4a4_act could not allocate its scratch buffer */
  GEMM_W4A4_ESCRATCH = -7     /* the call needs more scratch than quantize_w4a4_act_noalloc's
                                 fixed array (QUANTIZE_W4A4_NOALLOC_SCRATCH_BYTES) */
};

#define GEMM_W4A4_MAX_R 1024

/*
 * gemm_w4a4 — enqueue y = scaled_mma(act, wgt) * wcscale + bias + lora_act_in @ lora_up.
 *
 * act, ascales, wgt, wscales, wcscale, bias, out: required (non-NULL).
 * lora_act_in, lora_up: may be NULL only when R == 0 (no LoRA term).
 * M, N >= 1; K >= 16 with K % 16 == 0; 0 <= R <= GEMM_W4A4_MAX_R.
 * stream: a hipStream_t passed as void*; NULL selects the null stream.
 *
 * Every out[m][n] with m < M, n < N is overwritten; nothing else is written
 * and no input is modified. A plan whose tail runs its K in slices (see
 * gemm_w4a4_plan_t) first keeps the slices' float32 sums in out's first
 * rows; every element holds its result once the call's work on the stream
 * has finished. Results are deterministic: the same inputs give the same
 * bytes on every call (no atomics; slices are added in a fixed order). E4M3 NaN scale bytes
 * (0x7F, 0xFF) propagate NaN into every output their block touches.
 * Returns GEMM_W4A4_OK or one of the negative codes above.
 */
int gemm_w4a4(const uint8_t* act, const uint8_t* ascales,
              const uint8_t* wgt, const uint8_t* wscales,
              const float* wcscale, const float* bias,
              const uint16_t* lora_act_in, const uint16_t* lora_up,
              uint16_t* out, int M, int N, int K, int R, void* stream);

/*
 * gemm_w4a4_f16 — the same operation with the LoRA operands and the output in
 * IEEE binary16 instead of bfloat16 (the SVDQuant page runs its operator with
 * either 16-bit type, "c_dtype", sections 6.6 and 9.2):
 *   lora_act_in  uint16  [M, R]     binary16 bit patterns
 *   lora_up      uint16  [R, N]     binary16 bit patterns
 *   out          uint16  [M, N]     binary16 bit patterns (written), rounded to
 *                                   nearest even; magnitudes of 65520 and above
 *                                   become infinity
 * Every other argument, rule, alignment and return code is gemm_w4a4's.
 */
int gemm_w4a4_f16(const uint8_t* act, const uint8_t* ascales,
                  const uint8_t* wgt, const uint8_t* wscales,
                  const float* wcscale, const float* bias,
                  const uint16_t* lora_act_in, const uint16_t* lora_up,
                  uint16_t* out, int M, int N, int K, int R, void* stream);

/*
 * gemm_mxfp4 / gemm_mxfp4_f16 — the same operator with MXFP4 operands: E2M1
 * codes as above, but one UE8M0 scale per 32 consecutive k (value
 * 2^(b - 127), 0xFF = NaN; the DeepGEMM FP4 indexer page, "Step 0", pairs
 * E2M1 data with this block scale, applied by the matrix unit itself):
 *   ascales      uint8   [K/32, M]  UE8M0 bytes; scale of (m,k) is ascales[k/32][m]
 *   wscales      uint8   [K/32, N]
 * K >= 32 with K % 32 == 0; everything else (layouts, LoRA, affine, output
 * type bf16 or binary16, alignments, return codes) is gemm_w4a4's /
 * gemm_w4a4_f16's. No decode happens on the GPU: gfx950's scaled FP4 MFMA
 * consumes the packed bytes and the scale bytes as they are.
 */
int gemm_mxfp4(const uint8_t* act, const uint8_t* ascales,
               const uint8_t* wgt, const uint8_t* wscales,
               const float* wcscale, const float* bias,
               const uint16_t* lora_act_in, const uint16_t* lora_up,
               uint16_t* out, int M, int N, int K, int R, void* stream);
int gemm_mxfp4_f16(const uint8_t* act, const uint8_t* ascales,
                   const uint8_t* wgt, const uint8_t* wscales,
                   const float* wcscale, const float* bias,
                   const uint16_t* lora_act_in, const uint16_t* lora_up,
                   uint16_t* out, int M, int N, int K, int R, void* stream);

/*
 * Launch plan chosen by the solver for one problem size: which compiled tile
 * instance runs, and how that instance's LDS budget was solved — the ring
 * depth (stages of K in flight) and where the epilogue's first LoRA chunk and
 * per-column factors live — with the registers its code object uses. The
 * SVDQuant W4A4 on Blackwell page (section 7) shows what a miscounted buffer
 * in such a budget does: a silently shallower pipeline. Here the kernels carve
 * LDS from the same solved budget that these fields report. Pure host
 * arithmetic and table lookups (no HIP call), so it also runs without a GPU.
 */
typedef struct {
  int variant;        /* index of the compiled kernel instance */
  int block_m;        /* output rows per workgroup tile */
  int block_n;        /* output columns per workgroup tile */
  int block_k;        /* k per pipeline stage */
  int stages;         /* ring depth: LDS stages of K in flight, set by the budget solve */
  int waves_m;        /* wave grid inside a workgroup */
  int waves_n;
  int threads;        /* threads per workgroup */
  int lds_bytes;      /* LDS the instance uses: lds_ring_bytes + lds_side_bytes */
  int lds_stage_bytes;/* bytes of one ring stage (packed operands and their scales) */
  int lds_limit;      /* LDS available to one workgroup on gfx950 */
  int tiles_m;
  int tiles_n;
  int grid;           /* workgroups launched */
  int k_stages;       /* pipeline iterations over K */
  int lora_steps;     /* 16-deep LoRA MFMA steps (ceil(R/16)) */
  int occupancy;      /* workgroups of this instance per compute unit (LDS share = lds_limit / occupancy) */
  int policy;         /* budget solve: 0 deepest ring first, 1 whole side region first */
  int lora_place;     /* where the first 32 LoRA ranks and wcscale/bias wait for the epilogue:
                         0 nowhere: loaded by the epilogue and staged through the drained ring;
                         1 side region with wcscale/bias and the lora_act_in rows (lora_up in
                           registers held through the K-loop);
                         2 side region with the lora_up rows too.
                         Ranks past 32 always go through the drained ring. */
  int lds_ring_bytes; /* stages * lds_stage_bytes */
  int lds_side_bytes; /* side region beside the ring (0 when lora_place == 0) */
  int flavour;        /* kernel flavour the shape gets when every tensor is 16-byte aligned:
                         0 general, 1 fast, 2 fast with act-scale windows; -1 in variant_info */
  int vgprs;          /* vector registers a lane of that kernel (bf16 output) holds, architectural and
                         accumulation together, from its code object; -1 if unknown */
  int agprs;          /* of which accumulation registers */
  int sgprs;          /* scalar registers, same kernel */
  int regs_limit;     /* VGPR + AGPR a lane may hold at this occupancy (512 per SIMD lane, shared) */
  int k_groups;       /* waves sharing each wave tile, splitting every stage's k-steps between them
                         (threads = 64 * waves_m * waves_n * k_groups) */
  /* A split plan (the solver's choice only, tail_variant >= 0): the fields
   * above describe a first launch over the first M - tail_rows rows (whole
   * tile rows: tiles_m * block_m of them), and a second launch of instance
   * tail_variant, whose block_m divides the first one's, covers the last
   * tail_rows rows in tail_grid workgroups. Both run on the call's stream, in order, on
   * disjoint output rows. Not split: tail_variant -1, the others 0. */
  int tail_variant;
  int tail_rows;
  int tail_block_m;
  int tail_block_n;
  int tail_grid;
  /* K slices of the tail launch (1: it runs whole). Above 1, its workgroups
   * (tail_grid of them, counted with the slices) each run one slice of K and
   * write float32 sums into the first tail_splits * tail_rows * 2 rows of out,
   * rows the first launch writes later; a reduction launch adds the slices
   * into the last tail_rows rows. The three launches run on the call's stream
   * in the order slices, reduction, first launch; the call allocates nothing.
   * When the call's pointers do not allow the fast flavour the tail runs
   * whole, after the first launch. */
  int tail_splits;
} gemm_w4a4_plan_t;

/* Fill *plan for (M, N, K, R). Returns GEMM_W4A4_OK or GEMM_W4A4_EINVAL
 * (same size rules as gemm_w4a4; plan may not be NULL). */
int gemm_w4a4_plan(int M, int N, int K, int R, gemm_w4a4_plan_t* plan);

/* Number of compiled kernel instances, and the plan fields fixed by instance
 * `variant` (problem-size fields are zero). Returns GEMM_W4A4_EINVAL for an
 * unknown index. Used to check the solver against the compiled code objects. */
int gemm_w4a4_num_variants(void);
int gemm_w4a4_variant_info(int variant, gemm_w4a4_plan_t* plan);

/* The same three for the MXFP4 kernels (K % 32 == 0). */
int gemm_mxfp4_plan(int M, int N, int K, int R, gemm_w4a4_plan_t* plan);
int gemm_mxfp4_num_variants(void);
int gemm_mxfp4_variant_info(int variant, gemm_w4a4_plan_t* plan);

/* Operand formats and output types of gemm_w4a4_run / gemm_w4a4_plan_variant. */
enum { GEMM_W4A4_FMT_NVFP4 = 0, GEMM_W4A4_FMT_MXFP4 = 1 };

/*
 * gemm_w4a4_run — the same operator with every choice explicit, for callers
 * that pick the tiling per shape themselves (the solver's choice is a model;
 * this runs any compiled instance):
 *   format   GEMM_W4A4_FMT_NVFP4 (as gemm_w4a4) or GEMM_W4A4_FMT_MXFP4 (as gemm_mxfp4)
 *   out_f16  0: LoRA operands and output bfloat16; 1: binary16 (as the _f16 calls)
 *   variant  a compiled instance of that format, 0 <= variant < its
 *            num_variants, or -1 for the solver's choice
 * Every other argument, layout, rule and return code is the named entry
 * point's; an unknown format or variant returns GEMM_W4A4_EINVAL.
 */
int gemm_w4a4_run(int format, int out_f16, int variant,
                  const uint8_t* act, const uint8_t* ascales,
                  const uint8_t* wgt, const uint8_t* wscales,
                  const float* wcscale, const float* bias,
                  const uint16_t* lora_act_in, const uint16_t* lora_up,
                  uint16_t* out, int M, int N, int K, int R, void* stream);

/* The plan gemm_w4a4_run would follow for (format, variant, M, N, K, R);
 * variant -1 gives the solver's choice (the format's _plan call). */
int gemm_w4a4_plan_variant(int format, int variant, int M, int N, int K, int R,
                           gemm_w4a4_plan_t* plan);

/*
 * quantize_w4a4_act — the other half of an SVDQuant W4A4 layer (the SVDQuant
 * W4A4 on Blackwell page, section 1, calls gemm_w4a4 the compute-bound half):
 * from the bf16 activations x, the NVFP4 operand gemm_w4a4 consumes and the
 * rank-R LoRA input, in one pass over x.
 *
 *   x            uint16  [M, K]     bfloat16 bit patterns (read)
 *   lora_down    uint16  [R, K]     bfloat16 bit patterns, one rank per row (read);
 *                                   may be NULL iff R == 0
 *   act          uint8   [M, K/2]   written: two E2M1 codes per byte, low nibble = even k
 *   ascales      uint8   [K/16, M]  written: OCP E4M3FN scale of (m, k) at [k/16][m]
 *   lora_act_in  uint16  [M, R]     written: bfloat16 bits of sum_k x[m,k] * lora_down[r,k]
 *                                   (float32 accumulation, rounded to nearest even);
 *                                   may be NULL iff R == 0
 *
 * The pages fix these layouts (section 2; single-level scaling, section 3.1)
 * but not how a block's scale is chosen or its codes rounded. This library's
 * reading, per row and block of 16 consecutive k:
 *   - a block holding a NaN or an infinity gets scale byte 0x7F (NaN) and zero codes;
 *   - otherwise scale = E4M3FN nearest-even of max|x| / 6, saturating at 448;
 *   - code = sign bit of x | E2M1 magnitude of |x| / scale, nearest with ties
 *     to the even code, saturating at 6; a zero scale keeps only the sign bit.
 * Every rounding decision is exact (the same as on the real numbers).
 *
 * M >= 1; K >= 16 with K % 16 == 0; 0 <= R <= QUANTIZE_W4A4_MAX_R; every
 * tensor below 2^31 bytes. Alignment: x and lora_down 16 bytes, act 8,
 * lora_act_in 2. No output may overlap an input or another output
 * (GEMM_W4A4_EOVERLAP). Device pointers owned by the caller; the work is
 * enqueued on `stream` (one launch, or two when a 128-row instance splits K
 * with R > 0: the second adds the slices' partial sums; quantize_w4a4_act_plan
 * says which).
 *
 * Scratch: when few rows meet a long K, K is split over workgroups and
 * float32 partial sums go to a scratch buffer that the library allocates per
 * device and stream on the first call on that stream that needs it (or more
 * than it holds) and keeps until the process ends. That call allocates,
 * zeroes the buffer and synchronises the device before it enqueues anything
 * (GEMM_W4A4_ENOMEM if the allocation fails); every other call allocates and
 * synchronises nothing. Calls on different streams use different buffers, so
 * they may overlap. quantize_w4a4_act_noalloc never allocates. Other return
 * codes as for gemm_w4a4.
 */
#define QUANTIZE_W4A4_MAX_R 128
int quantize_w4a4_act(const uint16_t* x, const uint16_t* lora_down, uint8_t* act,
                      uint8_t* ascales, uint16_t* lora_act_in, int M, int K, int R,
                      void* stream);

/* The launch quantize_w4a4_act would make for (M, K, R): host only, nothing
 * enqueued. The instance follows the rank and, at R <= 32, the shape; K is
 * split over workgroups so that all row blocks' workgroups spread over the
 * compute units in one round (the device's count; 256 when no device is
 * current). */
typedef struct {
  int variant;          /* compiled producer instance */
  int wide;             /* 1: the waves of a workgroup share each span (lora_down tile in LDS) */
  int rank_tiles;       /* 16-rank tiles the instance covers (R <= 16 * rank_tiles) */
  int rows;             /* rows of x per workgroup */
  int threads;          /* threads per workgroup */
  int lds_bytes;        /* LDS per workgroup */
  int row_blocks;       /* ceil(M / rows) */
  int k_slices;         /* workgroups sharing a row block's K */
  int spans_per_slice;  /* 128-wide spans of K per slice */
  int grid;             /* workgroups of the first launch (row_blocks * k_slices) */
  int launches;         /* 2 when a wide kernel's slices are added by a second launch */
  long long scratch_bytes;  /* scratch the call needs (arrival counters + partial sums); 0 unsplit */
} quantize_w4a4_plan_t;

/* Fill *plan. Returns GEMM_W4A4_OK, or GEMM_W4A4_EINVAL for sizes
 * quantize_w4a4_act rejects or a NULL plan. */
int quantize_w4a4_act_plan(int M, int K, int R, quantize_w4a4_plan_t* plan);

/*
 * quantize_w4a4_act_noalloc — quantize_w4a4_act for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Same arguments, kernels and results as
 * quantize_w4a4_act; it calls no allocating routine.
 *
 * When K is split over several workgroups (few rows, long K), the kernels
 * keep float32 partial sums (and, for R <= 32, one arrival counter per 16
 * rows) in scratch memory; quantize_w4a4_act allocates that buffer on first
 * need, this entry
 * point uses a fixed device array of QUANTIZE_W4A4_NOALLOC_SCRATCH_BYTES
 * (4 KiB of counters + 16 MiB of partial sums) that each GPU holds until the
 * process ends. Both entry points split K only as far as 16 MiB of partial
 * sums allow; a call that would still need more returns GEMM_W4A4_ESCRATCH
 * with nothing enqueued. The counters are zero at load and every completed call
 * returns them to zero.
 *
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (concurrent streams, or host threads) race on it and must be ordered
 * by the caller. Return codes as for quantize_w4a4_act, plus
 * GEMM_W4A4_ESCRATCH.
 */
#define QUANTIZE_W4A4_NOALLOC_SCRATCH_BYTES (4096 + (16 << 20))
int quantize_w4a4_act_noalloc(const uint16_t* x, const uint16_t* lora_down, uint8_t* act,
                              uint8_t* ascales, uint16_t* lora_act_in, int M, int K, int R,
                              void* stream);

/* Static string for a return code (never NULL). */
const char* gemm_w4a4_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_W4A4_H */
