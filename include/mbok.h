/*
 * mbok.h -- C ABI of the Multi-Boolean-kernel (MBOK) linear layer for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation is the linear-layer product of a weight matrix stored as K
 * Boolean kernels with group scales:
 *
 *     W_hat = sum_{k=1..K} alpha_k (.) B_k,   B_k in {-1,+1}^{m x n},
 *     y     = W_hat . x      (decode, one token)
 *     Y     = X . W_hat^T    (several tokens)
 *
 * Sources (page title, then the section on that page):
 *   [RN]  "Highly Efficient and Effective LLMs with Multi-Boolean
 *         Architectures", Paper-Notes reading note (zhaoyang97.github.io),
 *         sections 关键设计 (key design: multi-kernel Boolean parameters,
 *         closed-form scale fit, group-wise scales), 消融实验 (ablation table:
 *         group size 128 is the usual choice), 训练策略 (initialisation by SVD or
 *         greedy search) and 局限与展望 (activations stay full precision).
 *   [GS]  the same paper's gist.science summaries (Italian, Dutch, Spanish),
 *         sections "Architetture Multi-Kernel" / "Successive SVID" /
 *         "Extracción Sucesiva": successive kernels are fitted to the residual
 *         of the previous ones.
 *
 * Conventions shared by every call
 * ---------------------------------
 *  - m = output features (rows of W), n = input features (columns of W).
 *    W is row-major [m, n]; x has n entries; y has m entries; X is row-major
 *    [T, ldx >= n]; Y is row-major [T, ldy >= m].
 *  - Scales: one alpha per (kernel k, output row i, group g) where group g is
 *    the 128 consecutive input columns 128g .. 128g+127 ([RN] group-wise scales,
 *    group size 128).  n must be a multiple of 128.
 *  - Sign encoding: bit 1 <-> +1, bit 0 <-> -1 ([GS] Dutch summary,
 *    Methodologie 1: a Boolean weight is -1/+1, equivalently FALSE/TRUE; here
 *    TRUE is bit 1 and means +1).  sign(0) and sign(-0.0) are +1.
 *  - All data pointers are DEVICE memory owned by the caller.  The library
 *    allocates nothing and every call only enqueues work on `stream` (a
 *    hipStream_t; NULL = the default stream) and returns without
 *    synchronising.  The one piece of global state is the static scratch of
 *    mbok_gemvt_noalloc (a fixed device array, its address cached per device).
 *  - Every argument check runs on the host before anything is enqueued, so an
 *    error return means nothing was launched and no output was touched.
 *    MBOK_ERR_HIP is returned when a launch itself fails (hipGetLastError).
 *  - Results are deterministic: the same inputs give the same output bits
 *    (no atomics, fixed reduction order).
 *
 * Packed layout MBOK_LAYOUT_L64 (what mbok_pack writes and mbok_gemv /
 * mbok_gemm read)
 * -------------------------------------------------------------------------
 *  m_pad = m rounded up to a multiple of 64, G = n / 128.
 *  The buffer has two regions:
 *
 *  1. sign bits, K * m_pad * n / 8 bytes, starting at byte 0.  It is a
 *     sequence of 16-byte chunks; chunk c holds the 128 signs of one
 *     (row i, group g, kernel k) with
 *         c = ((rb * G + g) * K + k) * 64 + r,   rb = i / 64,  r = i % 64.
 *     A chunk is four little-endian uint32 words; word w (0..3) covers
 *     columns 128g + 32w .. 128g + 32w + 31, and
 *         bit (8e + q) of word w  <->  column 128g + 32w + 4q + e
 *     for e in 0..3, q in 0..7.  Equivalently: byte 4w + e of the chunk,
 *     bit q, is column 128g + 32w + 4q + e.  So each 4-bit nibble of a word
 *     holds 4 columns spaced 4 apart (one signed-sum lookup in the decode
 *     kernel), and the 4 bits of 4 consecutive columns 4q..4q+3 sit at the
 *     same position q of the word's 4 bytes (one byte-select in the prefill
 *     unpack).  Rows m .. m_pad-1 are all-zero bits.
 *
 *  2. scales, starting at byte K * m_pad * n / 8 (a multiple of 1024):
 *     K * m_pad * G values of the descriptor's alpha dtype (fp32 or IEEE
 *     fp16), value index ((rb * G + g) * K + k) * 64 + r, i.e. in the same
 *     order as the chunks.  Scales of padding rows are 0.
 *
 *  So one (row block, group) holds K consecutive 1 KB sign planes of 64 rows,
 *  and 64 consecutive scales per plane: a wavefront of 64 lanes, one lane per
 *  row, reads one plane with one 16-byte load per lane (1 KB contiguous).
 */
#ifndef MBOK_H
#define MBOK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MBOK_GROUP 128      /* input columns per scale group */
#define MBOK_ROW_BLOCK 64   /* rows per packed row block */
#define MBOK_MAX_K 4        /* kernels per layer accepted by the library */
#define MBOK_MAX_T 65536    /* tokens per mbok_gemm call */

/* Status codes.  0 is success; errors are negative. */
enum {
  MBOK_OK = 0,
  MBOK_ERR_INVALID_ARG = -1, /* NULL pointer, unknown enum, bad leading dim */
  MBOK_ERR_SHAPE = -2,       /* m < 1, n < 128, n % 128 != 0, T out of range */
  MBOK_ERR_DTYPE = -3,       /* dtype not accepted by this call */
  MBOK_ERR_ALIGN = -4,       /* pointer or leading dimension misaligned */
  MBOK_ERR_HIP = -5,         /* the HIP runtime rejected a launch */
  MBOK_ERR_UNSUPPORTED = -6, /* K or group outside what the library runs */
  MBOK_ERR_INFEASIBLE = -7,  /* no kernel allocation fits the bit budget */
  MBOK_ERR_SCRATCH = -8      /* more scratch needed than the static scratch holds */
};

/* Element types. */
enum { MBOK_F32 = 0, MBOK_F16 = 1, MBOK_BF16 = 2 };

/* Packed layouts. */
enum { MBOK_LAYOUT_L64 = 1 };

/* Shape of one MBOK layer.  Fill it with mbok_desc_init. */
typedef struct mbok_desc {
  int32_t m;           /* output features, >= 1 */
  int32_t n;           /* input features, a positive multiple of 128 */
  int32_t K;           /* Boolean kernels, 1 .. MBOK_MAX_K */
  int32_t group;       /* always MBOK_GROUP */
  int32_t alpha_dtype; /* MBOK_F32 or MBOK_F16 */
  int32_t layout;      /* always MBOK_LAYOUT_L64 */
} mbok_desc;

/*
 * Describes one layer of K Boolean kernels with group-wise scales ([RN]
 * 关键设计: a weight matrix is the sum of K Boolean kernels, each with its own
 * scales, one scale per group of input columns; [RN] 消融实验: groups of 128).
 * Fills *d after checking the shape: 1 <= m <= 2^24, 128 <= n <= 2^20 with
 * n % 128 == 0, 1 <= K <= MBOK_MAX_K, alpha_dtype in {MBOK_F32, MBOK_F16}.
 * Host only.  Returns MBOK_OK, MBOK_ERR_INVALID_ARG (d NULL),
 * MBOK_ERR_SHAPE, MBOK_ERR_UNSUPPORTED (K) or MBOK_ERR_DTYPE.
 */
int mbok_desc_init(mbok_desc* d, int32_t m, int32_t n, int32_t K,
                   int32_t alpha_dtype);

/* Bytes of the packed buffer (both regions of MBOK_LAYOUT_L64).  Host only;
 * returns 0 for a NULL or invalid descriptor. */
size_t mbok_packed_bytes(const mbok_desc* d);

/* Bytes of the natural-order scale array alpha[K][m][n/128] that
 * mbok_residual_binarize writes and mbok_pack reads.  Host only; 0 for a NULL
 * or invalid descriptor. */
size_t mbok_alpha_bytes(const mbok_desc* d);

/*
 * Greedy residual binarization: the data-free extraction of the K kernels
 * from a floating-point weight ([RN] 训练策略: initialisation by greedy
 * search; [GS] successive kernels fitted to the residual; [RN] 关键设计: for
 * fixed signs the least-squares scale has a closed form).  Per (row, group),
 * in float64:
 *     R_0 = W
 *     for k = 1..K:
 *         B_k   = sign(R_{k-1})                  (0 and -0.0 map to +1)
 *         a     = mean over the group of |R_{k-1}|   (the LS-optimal scale)
 *         alpha = a rounded to nearest-even in the alpha dtype
 *         R_k   = R_{k-1} - alpha * B_k          (uses the rounded alpha)
 *
 *  W      device, fp32, row-major [m, ldw], ldw >= n (elements).
 *  signs  device, int8 [K][m][n] row-major, written with +1 / -1.
 *  alpha  device, [K][m][n/128] of d->alpha_dtype (natural order).
 *  flag   device int32 or NULL.  If W holds a NaN or an Inf the call stores 1
 *         there (it never stores 0: the caller clears it beforehand) and the
 *         outputs for the affected groups are unspecified.
 * Errors: INVALID_ARG (NULL, ldw < n), SHAPE/DTYPE/UNSUPPORTED from d,
 * ALIGN (W, signs or alpha not 16-byte aligned, ldw % 4 != 0), HIP.
 */
int mbok_residual_binarize(const mbok_desc* d, const float* W, int64_t ldw,
                           int8_t* signs, void* alpha, int32_t* flag,
                           void* stream);

/* Largest `rounds` accepted by mbok_refit. */
#define MBOK_MAX_REFIT_ROUNDS 64

/*
 * Alternating least-squares refit of K Boolean kernels and their scales for
 * the weight W they approximate ([RN] 关键设计, efficient scale optimisation:
 * with the Boolean matrices fixed the scales have a closed-form least-squares
 * solution, and signs and scales are optimised in turn).  Usually run on the
 * output of mbok_residual_binarize, before mbok_pack.  Per (row i, group g),
 * with w the 128 weights of the group and b_k its signs:
 *     repeat `rounds` times: scale step, sign step; then one scale step
 *     scale step: alpha = exact solution of (B^T B) alpha = B^T w, rounded
 *                 once to nearest-even in the alpha dtype; when the integer
 *                 K x K matrix B^T B is singular the scales are kept
 *     sign step:  each weight takes the signs of its nearest level
 *                 sum_k alpha_k b_k (float64 levels summed in k order and
 *                 float64 distances; a tie goes to the larger level, then to
 *                 the larger pattern index sum_k [b_k = +1] 2^k)
 * rounds = 0 only re-solves the scales.  With K = 1 nothing changes (the
 * least-squares scale of sign(w) is mean |w|).  Scales may come out
 * negative.
 *  W       device, fp32, row-major [m, ldw], ldw >= n (elements); read only.
 *  signs   device, int8 [K][m][n], read and overwritten in place with +1 /
 *          -1; an entry >= 0 is read as +1.
 *  alpha   device, [K][m][n/128] of d->alpha_dtype (natural order), read
 *          and overwritten in place.
 *  rounds  0 .. MBOK_MAX_REFIT_ROUNDS.
 * The scale step is exact (one rounding of the rational solution) whenever,
 * within each group, the nonzero weights' magnitudes lie within a factor 2^48
 * of one another; otherwise the solution is accurate to about 2^-100 before
 * its rounding.  NaN or Inf weights give unspecified outputs for their
 * groups (mbok_residual_binarize reports them).
 * Errors: INVALID_ARG (NULL, ldw < n, rounds out of range),
 * SHAPE/DTYPE/UNSUPPORTED from d, ALIGN (W, signs or alpha not 16-byte
 * aligned, ldw % 4 != 0), HIP.
 */
int mbok_refit(const mbok_desc* d, const float* W, int64_t ldw, int8_t* signs,
               void* alpha, int32_t rounds, void* stream);

/*
 * Residual energy of the greedy decomposition (the chain of
 * mbok_residual_binarize with d->K kernels) after k = 0..K kernels: the
 * residual approximation error that the kernel allocation weighs ([GS]
 * Italian summary, section "D. Allocazione Automatica dei Kernel").
 *     row_energy[k * m + i] = float64 nearest to sum_j R_k[i, j]^2
 *     layer_energy[k]       = float64 nearest to sum_i row_energy[k * m + i]
 * with R_0 = W and R_k the float64 residual after k kernels (the scales
 * rounded to d->alpha_dtype exactly as mbok_residual_binarize rounds them).
 * Because the greedy chain does not depend on how many kernels follow,
 * layer_energy[K'] is the error of the K'-kernel decomposition for every
 * K' <= K.  The sums are exact pair sums before their one rounding when a
 * row's squared residuals (and the layer's row energies) lie within a factor
 * of about 2^90 (2^48) of one another.
 *  W             device, fp32, row-major [m, ldw], ldw >= n; read only.
 *  row_energy    device, float64 [K + 1][m]; overwritten.
 *  layer_energy  device, float64 [K + 1]; overwritten.
 * Errors: INVALID_ARG (NULL, ldw < n), SHAPE/DTYPE/UNSUPPORTED from d, ALIGN
 * (W 16 bytes, ldw % 4, energies 8 bytes), HIP.
 */
int mbok_residual_energy(const mbok_desc* d, const float* W, int64_t ldw,
                         double* row_energy, double* layer_energy, void* stream);

/*
 * Number of kernels for each of L weights under a bit budget ([GS] Italian
 * summary, section "D. Allocazione Automatica dei Kernel": kernels per
 * weight chosen for an average bit budget from residual error and weight
 * size; the importance term needs data and is left out, so every weight
 * counts the same).  Host only, no GPU work.  Chooses K_l in 1..kmax with
 *     sum_l K_l * sizes[l] <= budget
 * minimising the exact sum of errors[l * kmax + K_l - 1]; among equal
 * errors the fewest bits, then the first K vector in lexicographic order.
 * The answer is exact (dynamic programming over exact error sums).
 *  L       number of weights, >= 1.
 *  sizes   host int64 [L], entries per weight (bits per kernel), each >= 1.
 *  errors  host float64 [L][kmax], errors[l * kmax + K - 1] = residual energy
 *          of weight l with K kernels (e.g. layer_energy[K] of
 *          mbok_residual_energy); finite and >= 0.
 *  kmax    1 .. MBOK_MAX_K.
 *  budget  total kernel-bits, e.g. floor(average kernels * sum of sizes).
 *  K_out   host int32 [L], written on success only.
 * Errors: INVALID_ARG (NULL, L < 1, kmax, sizes < 1, errors negative or not
 * finite, budget < 0), INFEASIBLE (sum of sizes > budget), UNSUPPORTED (more
 * than 2^22 partial allocations would be compared).
 */
int mbok_allocate_kernels(int32_t L, const int64_t* sizes, const double* errors,
                          int32_t kmax, int64_t budget, int32_t* K_out);

/* Largest number of power-iteration rounds accepted by mbok_svid_decompose. */
#define MBOK_MAX_SVID_ITERS 1000

/* Bytes of the workspace mbok_svid_decompose needs (float64 iterates and
 * partial sums).  Host only; 0 for a NULL or invalid descriptor. */
size_t mbok_svid_workspace_bytes(const mbok_desc* d);

/*
 * Successive sign-value-independent decomposition (SVID), the scale variant
 * of the [GS] summaries ("Riformulazione Booleana e SVID", "Successive
 * SVID", "Descomposición SVID"): W ~ sum_k B_k (.) (s_out^k s_in^k^T), where
 * for k = 1..K, with R_0 = W:
 *     B_k          = sign(R_{k-1})            (0 and -0.0 give +1)
 *     sigma, u, v  = the top singular triple of |R_{k-1}|, by `iters` rounds
 *                    of float64 power iteration from v = 1/sqrt(n)
 *     s_out^k      = sqrt(sigma) u, s_in^k = sqrt(sigma) v, each rounded once
 *                    to nearest-even in d->alpha_dtype
 *     R_k          = R_{k-1} - B_k (.) (s_out^k s_in^k^T)  (float64, with the
 *                    rounded vectors)
 * The residual is recomputed from W on every pass (never stored).  Power
 * iteration reaches the SVD's vectors when the ratio of the two largest
 * singular values of |R| is well below 1 (about 0.03 for trained-like
 * weights, so 16-32 rounds give float64 accuracy).  Sums run in a fixed
 * order: results are bit-reproducible.
 *  W          device, fp32, row-major [m, ldw], ldw >= n; read only.
 *  signs      device, int8 [K][m][n]; written with +1 / -1.
 *  s_out      device, [K][m] of d->alpha_dtype; written.
 *  s_in       device, [K][n] of d->alpha_dtype; written.
 *  iters      1 .. MBOK_MAX_SVID_ITERS.
 *  workspace  device, mbok_svid_workspace_bytes(d) bytes, 256-byte aligned;
 *             needs no initialisation; calls that may overlap need distinct
 *             workspaces.
 * Errors: INVALID_ARG (NULL, ldw < n, iters), SHAPE/DTYPE/UNSUPPORTED from
 * d, ALIGN (W and signs 16 bytes, ldw % 4, vectors 4 bytes, workspace 256
 * bytes), HIP.
 */
int mbok_svid_decompose(const mbok_desc* d, const float* W, int64_t ldw,
                        int8_t* signs, void* s_out, void* s_in, int32_t iters,
                        void* workspace, void* stream);

/*
 * Packs SVID kernels into MBOK_LAYOUT_L64: the sign bits as mbok_pack writes
 * them, and s_out^k[i] in the scale slot of every group of row i, kernel k.
 * (s_in is passed to mbok_svid_gemv separately.)
 *  signs   device int8 [K][m][n];  s_out  device [K][m] of d->alpha_dtype;
 *  packed  device, mbok_packed_bytes(d) bytes, fully overwritten.
 * Errors: INVALID_ARG, SHAPE/DTYPE/UNSUPPORTED, ALIGN (signs and packed 16
 * bytes, s_out 4 bytes), HIP.
 */
int mbok_svid_pack(const mbok_desc* d, const int8_t* signs, const void* s_out,
                   void* packed, void* stream);

/* Bytes of the workspace mbok_svid_gemv uses: 0 (the argument is kept for a
 * form that stages activations).  Host only. */
size_t mbok_svid_gemv_workspace_bytes(const mbok_desc* d);

/*
 * Decode product of the SVID representation ([GS] summaries: the product is
 * the Boolean one with x scaled per kernel and the output scaled per row):
 *     y[i] = sum_k s_out^k[i] * sum_j b_k[i, j] * s_in^k[j] * x[j]
 * s_in^k (.) x is formed in fp32 (exact for fp16 scales and bf16 x) and
 * split into four fp8 parts with one power-of-two scale per 32 columns, 4
 * bits each, so the matrix cores see 16 significant bits of each 32-column
 * word's largest value (MBOK_SVID_VARIANT=skinny: bf16 hi + lo parts, about
 * 2^-17 relative per value); the +-1 contractions accumulate in fp32 and
 * s_out applies in fp32.  Within 1e-5 of sum_k |s_out^k[i]| sum_j |s_in^k[j]
 * x[j]| on the workloads; a non-finite product s_in^k[j] x[j] makes every
 * output NaN.  Results are bit-reproducible.
 *  packed     device, the buffer of mbok_svid_pack.
 *  s_in       device [K][n] of d->alpha_dtype, 16-byte aligned.
 *  x          device, n values of x_dtype (MBOK_BF16 or MBOK_F32), 16-byte
 *             aligned.
 *  y          device fp32 [m]; overwritten.
 *  workspace  device pointer or NULL; unused (checked for 256-byte alignment
 *             when given).
 * Errors: INVALID_ARG (NULL), SHAPE/UNSUPPORTED from d, DTYPE (x_dtype),
 * ALIGN (packed, s_in, x 16 bytes, y 4 bytes, workspace 256 bytes), HIP.
 */
int mbok_svid_gemv(const mbok_desc* d, const void* packed, const void* s_in,
                   const void* x, int32_t x_dtype, float* y, void* workspace,
                   void* stream);

/*
 * Packs Boolean kernels and their scales into MBOK_LAYOUT_L64 (see the top
 * of this header): the storage form of the multi-kernel Boolean parameters
 * ([RN] 关键设计: K sign matrices and their group scales; [GS] Dutch
 * summary, Methodologie 1: a Boolean weight is -1/+1, i.e. FALSE/TRUE, so one
 * bit holds it).
 * Any +-1 signs are accepted, e.g. those of a finetuned model ([GS] Dutch
 * summary, Methodologie 3: the kernels are finetuned in the Boolean domain);
 * an entry >= 0 packs as bit 1 (+1) and < 0 as bit 0 (-1).
 *  signs   device int8 [K][m][n].
 *  alpha   device [K][m][n/128] of d->alpha_dtype.
 *  packed  device, mbok_packed_bytes(d) bytes; fully overwritten, padding
 *          included.
 * Errors: INVALID_ARG, SHAPE/DTYPE/UNSUPPORTED, ALIGN (16 bytes), HIP.
 */
int mbok_pack(const mbok_desc* d, const int8_t* signs, const void* alpha,
              void* packed, void* stream);

/*
 * Bytes of the workspace mbok_gemv uses for this shape: 0 when the call needs
 * none, which is the case for every shape with the default kernel (the
 * column-split kernel, selected for comparison with the environment variable
 * MBOK_GEMV_VARIANT=split, is the one that uses it).  Host only; 0 for a NULL
 * or invalid descriptor.
 */
size_t mbok_gemv_workspace_bytes(const mbok_desc* d);

/*
 * Decode product for one token ([RN] 关键设计: Wx splits into K Boolean
 * matrix-vector products, so each weight multiply becomes an add or a
 * subtract of an activation; [RN] 局限与展望: activations stay full
 * precision):
 *     y[i] = sum_k sum_g alpha_k[i,g] * sum_{j in group g} b_k[i,j] * x[j]
 * with fp32 accumulation.
 *  packed    device, MBOK_LAYOUT_L64 buffer of this descriptor.
 *  x         device, n values of x_dtype (MBOK_BF16 or MBOK_F32).
 *  y         device fp32 [m]; overwritten (not accumulated).
 *  workspace device, mbok_gemv_workspace_bytes(d) bytes, 256-byte aligned,
 *            or NULL (always allowed; ignored when the size is 0).  When used
 *            it receives the partial sums of column slices, which a second
 *            small kernel on the same stream adds in a fixed order; its
 *            contents need no initialisation and are meaningless after the
 *            call, and calls that may run at the same time (other streams)
 *            need distinct workspaces.
 * The default kernels keep one workgroup per compute unit and stream 16-row
 * tiles.  For bf16 x the products run on the matrix cores when a row holds at
 * least 8192 sign bits (K n >= 8192), the layer at least 2^25 (K m n), or
 * K = 4: signs as fp4 values (one of two per sign, a known offset removed per
 * group), each activation as an exact pair of fp8 parts with one power-of-two
 * scale per 32 columns, alpha applied per (row, group, kernel) in fp32.
 * Otherwise (and for fp32 x) signed-sum tables of x are built once and the
 * sign nibbles index them.
 * Non-finite x: with the table kernels a NaN or infinity propagates through
 * the fp32 sums; with the matrix-core kernel any NaN or infinite activation
 * makes every output NaN.
 * Errors: INVALID_ARG, SHAPE/UNSUPPORTED, DTYPE (x_dtype), ALIGN (packed and
 * x 16-byte aligned, y 4-byte aligned, workspace 256-byte aligned), HIP.
 */
int mbok_gemv(const mbok_desc* d, const void* packed, const void* x,
              int32_t x_dtype, float* y, void* workspace, void* stream);

/*
 * Bytes of the workspace mbok_gemvt uses for this shape (the partial column
 * sums of its row slices), 0 when it needs none.  Host only; 0 for a NULL or
 * invalid descriptor.
 */
size_t mbok_gemvt_workspace_bytes(const mbok_desc* d);

/*
 * Transposed decode product for one gradient vector, the activation gradient
 * of the layer (the [GS] summaries' Boolean-domain training propagates
 * gradients through the Boolean weights; [RN] 关键设计: the product splits
 * into K Boolean products):
 *     dx[j] = sum_i sum_k alpha_k[i, j/128] * b_k[i, j] * g[i]
 * Each term alpha_k[i, .] * g[i] is formed in fp32; the sums are fp32.
 *  packed    device, MBOK_LAYOUT_L64 buffer of this descriptor (the same
 *            buffer mbok_gemv reads).
 *  g         device, m values of g_dtype (MBOK_BF16 or MBOK_F32).
 *  dx        device fp32 [n]; overwritten (not accumulated).
 *  workspace device, mbok_gemvt_workspace_bytes(d) bytes, 256-byte aligned,
 *            or NULL.  With NULL one workgroup per column group walks all
 *            rows (correct, slower); with the workspace the rows are split
 *            into slices whose partial sums a second kernel adds in a fixed
 *            order.  Its contents need no initialisation; calls that may run
 *            at the same time need distinct workspaces.
 * Errors: INVALID_ARG (NULL), SHAPE/UNSUPPORTED from d, DTYPE (g_dtype),
 * ALIGN (packed 16 bytes, g and dx 4 bytes, workspace 256 bytes), HIP.
 */
int mbok_gemvt(const mbok_desc* d, const void* packed, const void* g,
               int32_t g_dtype, float* dx, void* workspace, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): mbok_gemvt
 * with its workspace replaced by the library's static scratch, a file-scope
 * device array of mbok_gemvt_scratch_bytes() = 512 KiB per device, held until
 * the process ends.  Same kernels, same slicing and the same output bits as
 * mbok_gemvt with a workspace.  The call allocates nothing: on its first call
 * on a device it looks up that device's address of the array
 * (hipGetSymbolAddress, with the caller's current device) and caches it.
 *  packed, g, g_dtype, dx, stream: as for mbok_gemvt.
 * Every call on one GPU shares that GPU's scratch: calls that may overlap in
 * time on the same GPU (different streams, different host threads) race and
 * must be serialised by the caller.  The scratch needs no initialisation
 * (every partial sum is written before it is read).
 * Errors: as mbok_gemvt; SCRATCH when the shape needs more than the static
 * scratch (no shape the descriptor accepts does); HIP when the device or the
 * array's address cannot be queried, or a launch fails.
 */
size_t mbok_gemvt_scratch_bytes(void);
int mbok_gemvt_noalloc(const mbok_desc* d, const void* packed, const void* g,
                       int32_t g_dtype, float* dx, void* stream);

/*
 * The same product for T tokens ([RN] 关键设计: the layer's product is the sum
 * of its K Boolean products, scaled per group; [RN] 局限与展望: activations
 * stay full precision):  Y[t, i] = sum_j W_hat[i, j] * X[t, j].
 * T = 1 runs the decode kernel of mbok_gemv (without a workspace).  T = 2,
 * and T = 3..6 on layers of at least 2^26 sign bits (K m n), run matrix-core
 * forms of that kernel for several tokens (signs as fp4 operands, each bf16
 * activation as two exact fp8 parts with one power-of-two scale per 32
 * columns, alpha applied per group in fp32: within ~1e-6 of the bound
 * sum_j |W_hat_ij| |X_tj| on Gaussian activations; bit-exact for small
 * integer activations and power-of-two scales).  The other T <= 16 run the
 * weight-streaming few-token kernel (exact fp32 scaling of +-1 products).  A
 * non-finite activation of token t makes row t of Y NaN on the matrix-core
 * paths (IEEE propagation elsewhere).  T > 16 is the prefill GEMM: each tile of W_hat is formed
 * as sum_k alpha_k * b_k in fp32, rounded to bf16 (nearest-even) in LDS, and
 * contracted with the bf16 X tile on the matrix cores with fp32 accumulation.
 *  X        device bf16 [T, ldx], ldx >= n, ldx % 8 == 0.
 *  Y        device fp32 [T, ldy], ldy >= m; overwritten.
 *  T        1 .. MBOK_MAX_T.
 * Errors: INVALID_ARG (NULL, ldx < n, ldy < m), SHAPE (T), DTYPE (x_dtype
 * other than MBOK_BF16), ALIGN (packed/X 16 bytes, ldx % 8, Y 4 bytes), HIP.
 */
int mbok_gemm(const mbok_desc* d, const void* packed, const void* X,
              int32_t x_dtype, int64_t T, int64_t ldx, float* Y, int64_t ldy,
              void* stream);

/*
 * mbok_gemm with the prefill weights carried to 16 significant bits ([RN]
 * 关键设计: W_hat x is the sum of the K scaled Boolean products, each weight
 * exactly sum_k alpha_k b_k; carrying that value to the matrix cores needs
 * more than bf16's 8 significant bits).  Same arguments, checks, errors and
 * output layout as mbok_gemm; T = 1 runs the same kernel as mbok_gemm, and
 * T = 2..16 always the weight-streaming few-token kernel (its products are
 * fp32-exact per scale).  For T > 16
 * each level v = sum_k +-alpha_k is formed in fp32 and split as
 * v = hi + lo with hi = bf16(v) and lo = bf16(v - hi), so |v - hi - lo| <=
 * 2^-16 |v|.  Two products run on `stream`: Y = X . HI^T, then Y += X . LO^T
 * (two launches, about twice the time and one extra read of Y).  Per output,
 * |Y - Y_exact| stays far below 1e-3 * sum_j |W_hat_ij| |X_tj| for any X
 * (2^-16 from the weights plus fp32 accumulation), where mbok_gemm's
 * one-term bf16 levels allow up to 2^-8 per weight.  The result is exactly
 * the fp64 product when every level has at most 16 significant bits (power-
 * of-two scales within 15 binades of each other) and the activations and sums
 * are small integers.
 */
int mbok_gemm_precise(const mbok_desc* d, const void* packed, const void* X,
                      int32_t x_dtype, int64_t T, int64_t ldx, float* Y,
                      int64_t ldy, void* stream);

/* Static description of a status code ("unknown status" for others). */
const char* mbok_status_str(int status);

/* Library version, e.g. "mbok 0.1.0 gfx950". */
const char* mbok_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MBOK_H */
