/*
 * sync_overlap.h -- C ABI of libsync_overlap.so: one GPU's share of a
 * chunk-overlapped collective GEMM on MI355X (gfx950).
 *
 * Sources for what the calls compute:
 *   [SYN-S] "Syncopate: Efficient Multi-GPU AI Kernels via Automatic
 *           Chunk-Centric Compute-Communication Overlap", paper summary page
 *           (awesome-system-papers), sections "Core method" (paper sec. 5.1,
 *           5.2, Fig. 6, Fig. 7) and "Experiments" (paper sec. 6.1, Fig. 8-9).
 *   [SYN-A] the same paper's abstract (arXiv 2601.20595 catalogue record).
 *   [SYN-R] the pith.science review page of that paper: captions of Fig. 3-7.
 *   [ENT]   "Entwine" abstract (arXiv 2609.11562, arxivdaily page).
 *
 * The pages pose the problem as a chunk schedule given together with a local
 * tile kernel [SYN-A]: the caller describes the chunk plan with sync_plan(); the tile
 * kernel is this library's persistent bf16 MFMA GEMM (or the ring-attention
 * step), whose tile traversal the plan reorders [SYN-S, Fig. 6] and whose
 * tiles wait in-kernel on per-chunk ready flags (AG) or raise per-chunk done
 * flags in send order (RS) [SYN-S "Core method"; ENT].  One GPU stands in for
 * every peer: the peers' shards sit in a separate HBM region and a copy agent
 * stages them in (SDMA engine, or load/store on dedicated CUs) [SYN-S, Fig. 7].
 *
 * Conventions for every call:
 *   - Return value: SYNC_OK (0) or a negative SYNC_E* code; on error,
 *     sync_last_error() returns a thread-local message.  No call aborts.
 *   - Device pointers are plain HIP device addresses owned by the caller and
 *     must be 16-byte aligned.  Host pointers are marked "host".
 *   - Streams are hipStream_t passed as void*; NULL means the null stream.
 *   - Launch calls are stream-ordered and asynchronous: SYNC_OK means the work
 *     was enqueued on `compute`.  Device-side failures (a wait that timed
 *     out) are read afterwards with sync_workspace_status().  The `copy`
 *     stream argument of the launch calls is reserved and unused: every
 *     backend runs on `compute` (the SDMA backend also on the engines).
 *   - All matrices are row-major.  bf16 = IEEE bfloat16 bit patterns.
 */
#ifndef SYNC_OVERLAP_H
#define SYNC_OVERLAP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
enum {
  SYNC_OK = 0,
  SYNC_EINVAL = -1,       /* bad argument: null/misaligned pointer, bad descriptor */
  SYNC_EUNSUPPORTED = -2, /* valid plan but no kernel variant for it (shape, tile) */
  SYNC_EHIP = -3,         /* a HIP runtime call failed; message holds its string */
  SYNC_ETIMEOUT = -4,     /* a device-side chunk wait ran past its time limit */
  SYNC_ENOMEM = -5,       /* host or device allocation failed */
  SYNC_ENODEV = -6        /* no usable gfx950 device */
};

/* ---- plan descriptor --------------------------------------------------- */
enum { SYNC_OP_AG_GEMM = 1, SYNC_OP_GEMM_RS = 2, SYNC_OP_RING_ATTN = 3, SYNC_OP_HEAD_ATTN = 4 };
enum { SYNC_PAT_RING = 0, SYNC_PAT_EXPLICIT = 1, SYNC_PAT_HIER_SWIZZLE = 2, SYNC_PAT_MESH = 3 };
enum { SYNC_ORDER_ROW_MAJOR = 0, SYNC_ORDER_CHUNK_MAJOR = 1, SYNC_ORDER_SWIZZLED = 2 };
enum { SYNC_B_KN = 0, SYNC_B_NK = 1 };      /* B as [k][n], or [n][k] (Linear weight) */
enum { SYNC_DTYPE_F32 = 0, SYNC_DTYPE_BF16 = 1 };

/*
 * A chunk plan [SYN-S "Core method", paper sec. 5.1: communication as P2P or
 * collective operations on chunks, each a block of a logical tensor holding
 * one or more tiles; ring is one of the patterns; plans may be user-written
 * or instantiated from templates].
 *
 * GEMM ops: C[m][n] = A[m][k] . B.  The chunked tensor is A (AG) or C (RS),
 *   split into `world` row shards of m/world rows, each cut into `split`
 *   sub-chunks by floor bounds: chunk c = w*split + q covers rows
 *   [w*R + floor(q*R/split), w*R + floor((q+1)*R/split)), R = m/world.
 * RING_ATTN: m = query rows Sq, n = tokens per KV block, k = head dim d;
 *   the chunked tensors are K and V ([world*n][heads_kv][d]).
 * HEAD_ATTN (head-parallel attention, the receive side of the all-to-all
 *   that turns sequence shards into head shards): n = tokens each peer
 *   sends, m = world*n (every token is a query), k = head dim; heads_q and
 *   heads_kv are this rank's head group.  The chunked tensors are Q, K and V
 *   ([world*n][heads][d]); block w comes from peer w.
 * Ring order (pattern RING, direction d = ring_dir):
 *   AG / attention: the shard consumed at step s is (rank - d*s) mod world
 *   (step 0 is the local shard); RS: the shard sent at step s is
 *   (rank - d*(s+1)) mod world (own shard last).  EXPLICIT: explicit_order
 *   (host, `world` entries, a permutation) lists shards in that order.
 *   HIER_SWIZZLE [SYN-S sec. 5.1 names hierarchical swizzles among the
 *   patterns a plan expresses]: ranks form world / hier_group groups of
 *   hier_group consecutive ranks; rank r = G*g + l takes at step a*g + b the
 *   shard ((G + a) mod (world/g))*g + (l + b) mod g: its own group first,
 *   then every group in turn, the ranks of a group pulling from distinct
 *   peers at every step; RS sends in the reverse of that order (own shard
 *   last).  MESH: the RING step order, but every peer's link runs at once:
 *   sub-chunk q of every shard is at position q*world + step(shard).
 * Tiles: tile t = i*tiles_n + j covers C rows [i*tile_m, ..) and columns
 *   [j*tile_n, ..) (attention: work item t = i*heads_q + h).  A tile depends
 *   on every chunk its rows meet (RING_ATTN: on every chunk; HEAD_ATTN: on
 *   the chunks holding its query rows); its key is the last (AG, attention) /
 *   first (RS) position among them.  Tile order [SYN-S, paper sec. 5.2, Fig. 6; ENT]:
 *   ROW_MAJOR (t ascending), CHUNK_MAJOR (key, i, j) or SWIZZLED
 *   (key, i / group_m, j, i).
 */
typedef struct {
  int32_t op;             /* SYNC_OP_* */
  int32_t world;          /* W >= 1 */
  int32_t rank;           /* 0 <= rank < W */
  int32_t ring_dir;       /* +1 or -1 */
  int64_t m, n, k;
  int32_t pattern;        /* SYNC_PAT_* */
  int32_t split;          /* 1 <= split <= rows per shard */
  const int32_t* explicit_order; /* host; read only during sync_plan() */
  int32_t tile_m, tile_n; /* GEMM tile (kernel variants: 256x256, 256x128, 128x128); attention: tile_m query rows */
  int32_t tile_order;     /* SYNC_ORDER_* */
  int32_t group_m;        /* SWIZZLED group height in tile rows; 0 = 4 */
  int32_t local_resident; /* 1: the rank's own shard is already in place (AG, attention) */
  int32_t heads_q, heads_kv; /* attention ops only; heads_q % heads_kv == 0 */
  int32_t b_layout;       /* SYNC_B_KN or SYNC_B_NK (GEMM ops) */
  const int64_t* shard_rows; /* host, GEMM ops, read only during sync_plan(): NULL = m / world rows
                                per shard; else world positive row counts summing to m, shard w
                                holding rows [sum of the counts before w, + shard_rows[w]) (an
                                all-to-all's receive side: peer w sends shard_rows[w] tokens) and
                                split <= the smallest count */
  int32_t hier_group;     /* HIER_SWIZZLE: ranks per group, dividing world; other patterns: 0 */
  int32_t reserved[1];    /* must be zero */
} sync_plan_desc;

typedef struct sync_plan_s* sync_plan_t;

/* Builds a plan on the CPU (no GPU needed).  *out is owned by the caller and
 * released with sync_plan_destroy().  The plan is immutable and may be shared
 * between threads.  EINVAL for an invalid descriptor. */
int sync_plan(const sync_plan_desc* desc, sync_plan_t* out);

/* Frees a plan and its device copies.  Only after every call using it has
 * completed on the device. */
void sync_plan_destroy(sync_plan_t plan);

typedef struct {
  int32_t num_chunks;  /* C = world * split */
  int32_t num_tiles;   /* T = tiles_m * tiles_n */
  int32_t tiles_m, tiles_n;
  int64_t num_deps;    /* total (tile, chunk) dependency pairs */
} sync_plan_info;

int sync_plan_get_info(sync_plan_t plan, sync_plan_info* out);

/* Caller-owned host arrays; a NULL member is skipped.  Sizes from
 * sync_plan_get_info: chunk_begin[C+1], chunk_pos[C], arrival[C] (chunk id
 * at each position), resident[C], tiles_in[C] (tiles per chunk),
 * tile_order[T], tile_key[T] (by tile id), dep_ptr[T+1], dep_idx[num_deps],
 * inv_ptr[C+1], inv_idx[num_deps]. */
typedef struct {
  int64_t* chunk_begin;
  int32_t* chunk_pos;
  int32_t* arrival;
  int32_t* resident;
  int32_t* tiles_in;
  int32_t* tile_order;
  int32_t* tile_key;
  int64_t* dep_ptr;
  int32_t* dep_idx;
  int64_t* inv_ptr;
  int32_t* inv_idx;
} sync_plan_tables;

int sync_plan_export(sync_plan_t plan, sync_plan_tables* out);

/* ---- copy agent configuration ------------------------------------------ */
/* Backends [SYN-S "Core method", paper sec. 5.2, Fig. 7: the same plan lowers
 * to a copy engine or to load/store on dedicated SMs, both signalling through
 * global-memory flags]:
 *   PRESET      no copy; every chunk is taken as present (compute-only; the
 *               caller provides the whole input)
 *   SDMA        the chunks move on the SDMA engines, queued through HSA
 *               (hsa_amd_memory_async_copy_on_engine; copy_teams engines, 1
 *               if 0).  On `compute` a one-workgroup gate kernel fixes the
 *               call's epoch and opens the call's gate signal, which every
 *               copy waits for; once every piece of a chunk's data copy has
 *               landed, an engine copies the epoch into the chunk's ready
 *               flag; the compute
 *               kernel follows on `compute`, on every CU (copy-only: a join
 *               kernel that waits for every flag).  `copy` is unused.  The
 *               host may wait (bounded) for the copies of the call made 16
 *               calls earlier on the device before queueing new ones.
 *   CU          the call is ONE kernel launch on `compute`: its first
 *               copy_cus x (compute workgroups per CU) workgroups copy, the
 *               rest compute; `copy` is unused.  Copy workgroups are spread
 *               evenly over the XCDs and are resident before any compute
 *               workgroup.
 *   HOST_GATED  withdrawn: every call returns EUNSUPPORTED.  (It queued
 *               stream-ordered runtime copies beside the persistent kernel;
 *               the runtime does not start such a copy while that kernel
 *               runs.)  The value stays reserved.  Failure-path tests use
 *               SYNC_RUN_WITHHOLD instead.
 *   COLOCATED   one launch on `compute` whose compute workgroups also copy; no
 *               CUs are set aside [SYN-S Fig. 7: load/store by the compute SMs
 *               themselves].  AG and attention: every workgroup first copies
 *               its share of each chunk and then computes.  GEMM-RS: every
 *               workgroup stores its tiles and then joins the copy-out, chunk
 *               by chunk in send order.
 *   CU and COLOCATED copy each chunk with 32-bit offsets: every chunk of a
 *               copied tensor (its rows x row bytes) must be under 2 GiB,
 *               else EUNSUPPORTED.
 *   EPILOGUE    GEMM-RS only: no copy pass at all; the epilogue of every tile
 *               stores it both into C and, row by row, into its chunk's send
 *               slot in `staging`, and the tile that completes chunk c raises
 *               sent[c] with done[c] [SYN-S Fig. 7: communication by the
 *               compute SMs' own stores; Entwine abstract: output handed to
 *               communication as the tiles produce it].  C may be NULL
 *               here: the send slots are then the only output.  Needs every
 *               tile inside one chunk (chunk bounds on tile rows) and
 *               m x n x (element size) below 2 GiB, else EUNSUPPORTED. */
enum { SYNC_COPY_PRESET = 0, SYNC_COPY_SDMA = 1, SYNC_COPY_CU = 2, SYNC_COPY_HOST_GATED = 3, SYNC_COPY_COLOCATED = 4,
       SYNC_COPY_EPILOGUE = 5 };

/* mode bits for sync_copy_cfg.flags */
enum {
  SYNC_RUN_COPY_ONLY = 1,    /* run only the copy (copy-only timing); AG and attention */
  SYNC_RUN_COMPUTE_ONLY = 2, /* run only the compute kernel, with the workgroups the CU split
                                leaves it (CU backend) or all CUs, every chunk taken as present */
  SYNC_RUN_TIMED = 4,        /* record device events around the call's kernel launch on the
                                compute stream; read with sync_read_timings() */
  SYNC_RUN_WITHHOLD = 8,     /* CU backend, AG and attention (failure-path tests): chunk
                                cfg.withhold_chunk (-1: every non-resident chunk) is neither
                                copied nor flagged, so the waits for it expire after timeout_ns,
                                exactly the tiles that read it stay unwritten, and the call
                                reports SYNC_ETIMEOUT naming it through sync_workspace_status */
  SYNC_RUN_TRACE = 16        /* GEMM calls: record per-tile and per-chunk device wall-clock
                                stamps in the workspace; read with sync_trace_export() */
};

typedef struct {
  int32_t backend;          /* SYNC_COPY_* */
  int32_t copy_cus;         /* CU backend: CUs given to the copy role, 8..128, multiple of 8 */
  uint64_t timeout_ns;      /* bound on every device-side wait; 0 = 2 s */
  const uint32_t* host_gates; /* reserved (the withdrawn HOST_GATED backend); ignored */
  int32_t flags;            /* SYNC_RUN_* bits */
  int32_t copy_streaming;   /* CU and COLOCATED backends: 1 = non-temporal loads/stores in the copy
                               role; 0 = plain */
  int32_t withhold_chunk;   /* SYNC_RUN_WITHHOLD only: the chunk left out, or -1 for all */
  int32_t copy_teams;       /* SDMA backend: engines used, at most max(number of chunks, 16) and
                               the engines available (copied chunk i goes to engine i mod
                               copy_teams; with E engines for C < E copied chunks, every chunk
                               is cut into floor(E / C) row pieces on distinct engines and its
                               flag is written once all of them have landed).  CU backend: chunks in flight at once; the copy workgroups split
                               into this many teams, team t taking every copy_teams-th copied
                               chunk from the t-th (copy-out: in send order, each team waiting
                               for its chunk's done flag).  0 or 1 = one chunk after another
                               (ring arrival); the number of copied chunks = all at once (pulls
                               from every peer in parallel, as over a full xGMI mesh). */
  int32_t copy_kslices;     /* AG-GEMM with the CU or COLOCATED backend: every chunk
                               moves as this many column blocks (K-slices) of its rows, slice 0
                               of every chunk first, each slice with its own ready flag; a tile
                               starts on slice 0 of its rows and waits in-kernel for slice h
                               just before it loads that K range, so tiles of late chunks start
                               early.  The chunk plan, dependency table and tile order are
                               unchanged.  0 or 1 = whole chunks; at most 8, with K/64 at least
                               4 x copy_kslices.  Other ops and backends: 0 or 1. */
  float copy_link_gbps;     /* CU backend: 0 = copy at the copy workgroups' own speed; else each
                               copy team stands for one link of this many GB/s (1e9 B/s, in
                               [1, 10000]) and delivers an item (chunk or K-slice; RS: a chunk of
                               C) no earlier than the link, free from its previous item and from
                               the moment the item may start, has carried its bytes (e.g. 153
                               for one xGMI link of an MI355X node: copy_teams = 1 paces a ring,
                               7 teams seven links at once) */
  int32_t copy_lead_slice;  /* AG-GEMM, CU backend, copy_kslices > 1: L in [1, copy_kslices] = the
                               first L K-slices of each copied chunk are copied by the compute
                               workgroups whose first tile reads that chunk (each a share of its
                               rows, published together), before they start it; the copy
                               workgroups move the other slices, and every slice of chunks no
                               first tile reads.  L = copy_kslices: those workgroups copy the
                               whole chunk, the per-tile co-located form.  0 = the copy
                               workgroups move every slice, as with COPY_ONLY (nothing
                               computes).  Not with pacing. */
} sync_copy_cfg;

/* ---- workspace ---------------------------------------------------------- */
/* Device scratch for flags, counters, the epoch and the error word.  Owned by
 * the caller, at least sync_workspace_size() bytes, 256-byte aligned.  Calls
 * on one workspace must be ordered (one stream, or joined streams); two calls
 * that may overlap in time race on it. */
size_t sync_workspace_size(sync_plan_t plan);

/* Zeroes the workspace with a fill kernel on `stream` and puts the plan's
 * tables on the current device if they are not there yet.  Call once after
 * allocation, and again after a call reported a device-side timeout (the
 * error word is sticky: later waits give up at once).  Between calls nothing
 * is cleared: each call's kernel takes the next epoch from the workspace and
 * its last workgroup stores it, so a call is exactly one launch on the
 * compute stream with the CU backend, and replaying a captured call is
 * valid.  First waits on the host (bounded; SYNC_ETIMEOUT) until every SDMA
 * copy queued on this device has completed, so that no flag write of an
 * earlier call lands after the fill. */
int sync_workspace_init(sync_plan_t plan, void* ws, void* stream);

/* Trace of the last SYNC_RUN_TRACE GEMM call on a workspace (waits for
 * `stream`).  Caller-owned arrays, any of which may be NULL; times in ns of the
 * device wall clock, relative to the earliest stamp of the call; -1 where
 * nothing was recorded (a tile that was skipped, a resident chunk, or a chunk
 * copied by SDMA).
 *   tile_wait_begin[T], tile_wait_end[T], tile_end[T]: when the workgroup took
 *     tile t, when its chunk waits were over (compute starts), and when its
 *     stores (and RS completion) were issued;
 *   tile_xcc[T]: XCD that ran the tile; tile_slot[T]: position p in the
 *     traversal at which it was taken (order[p] == t);
 *   chunk_ready[C]: AG: the copy role raised the chunk's ready flag; RS: the
 *     GEMM raised the chunk's done flag;  chunk_sent[C]: RS copy-out done. */
typedef struct {
  int64_t* tile_wait_begin;
  int64_t* tile_wait_end;
  int64_t* tile_end;
  int32_t* tile_xcc;
  int32_t* tile_slot;
  int64_t* chunk_ready;
  int64_t* chunk_sent;
} sync_trace;

int sync_trace_export(sync_plan_t plan, const void* ws, void* stream, sync_trace* out);

/* Synchronises `stream`, then reads the workspace error word.  Returns
 * SYNC_OK, or SYNC_ETIMEOUT with *err_chunk (may be NULL) = the chunk whose
 * wait expired first.  ws == NULL reads the static scratch of the current
 * device (the last sync_ag_gemm_noalloc call there). */
int sync_workspace_status(const void* ws, void* stream, int32_t* err_chunk);

/* ---- launch calls --------------------------------------------------------- */
/* AG-GEMM share [SYN-S "Experiments", paper sec. 6.1, Fig. 8: AG-GEMM;
 * "Core method": tiles wait until the chunks they consume have arrived].
 *   a_peer  bf16 [m][k]: every shard at its natural rows (stands in for the
 *           peers' memory); read-only.
 *   a_local bf16 [m][k]: the resident shard's rows are filled by the caller;
 *           the copy agent writes every other chunk's rows (PRESET: the caller
 *           fills all rows).
 *   b       bf16, [k][n] (SYNC_B_KN) or [n][k] (SYNC_B_NK).
 *   c       [m][n], c_dtype fp32 or bf16 (round to nearest even).
 * Kernel constraints (else EUNSUPPORTED): k % 64 == 0, n % 8 == 0, tile
 * (tile_m, tile_n) in {(256,256), (256,128), (128,128)}. */
int sync_ag_gemm(sync_plan_t plan, const sync_copy_cfg* cfg, const void* a_peer, void* a_local,
                 const void* b, void* c, int32_t c_dtype, void* ws, void* compute, void* copy);

/* AG-GEMM share for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same call as sync_ag_gemm (same arguments, kernels and result), except
 * that its workspace is the library's static device scratch, a 1 MiB array
 * that every GPU the library runs on holds until the process ends, and that
 * it calls no hipMalloc, hipFree or other allocating routine:
 *   - cfg must be non-NULL; backend PRESET, CU or COLOCATED (SDMA needs
 *     signals: EUNSUPPORTED); no SYNC_RUN_TIMED or SYNC_RUN_TRACE
 *     (EUNSUPPORTED); other cfg fields as for sync_ag_gemm.
 *   - The plan's tables must already be on the device: any earlier
 *     sync_workspace_init or launch call with this plan on the current device
 *     put them there (else EINVAL).
 *   - The plan's workspace (sync_workspace_size less its trace area) must fit
 *     in 1 MiB (else EINVAL), e.g. up to ~1000 chunks.
 *   - Each call first clears the part of the scratch it uses with a fill
 *     kernel on `compute` (stream-ordered, so the call can be captured), then
 *     launches as sync_ag_gemm does.  The scratch keeps the last call's
 *     contents; sync_workspace_status(NULL, stream, &chunk) reads its error
 *     word (a device-side timeout of the last call).
 *   - Every call on one GPU shares that GPU's scratch: calls that may overlap
 *     in time on one GPU (other streams, other threads) race on it; order
 *     them on one stream. */
int sync_ag_gemm_noalloc(sync_plan_t plan, const sync_copy_cfg* cfg, const void* a_peer, void* a_local,
                         const void* b, void* c, int32_t c_dtype, void* compute);

/* GEMM-RS share [SYN-S "Experiments": GEMM-RS; ENT: tiles reordered so output
 * for communication is produced at a steady pace; SM-based fine-grained
 * communication].  The GEMM visits tiles in send order; when the last tile of
 * chunk c is stored it raises done[c]; the copy workgroups (CU or COLOCATED
 * backend; SDMA: not supported, EUNSUPPORTED) wait for done[c] in send order and copy the
 * chunk's rows of c into `staging`, slot p = chunk arrival[p] (slots packed
 * back to back in send order).
 *   a bf16 [m][k]; b bf16 as in sync_ag_gemm; c and staging [m][n] c_dtype.
 * PRESET: the GEMM alone (done flags raised, no copy-out). */
int sync_gemm_rs(sync_plan_t plan, const sync_copy_cfg* cfg, const void* a, const void* b, void* c,
                 int32_t c_dtype, void* staging, void* ws, void* compute, void* copy);

/* GEMM-RS share with its reduce-scatter step [SYN-S "Experiments", paper
 * sec. 6.1: GEMM-RS; in a ring reduce-scatter each rank adds its own partial
 * result to the partial sum it receives and forwards the total].  As
 * sync_gemm_rs with the EPILOGUE backend and fp32 C, plus
 *   partials fp32 [m][n]: the partial sums arriving from the ring predecessor,
 *            at C's row positions (read-only);
 * staging slot p then holds C + partials over the rows of chunk arrival[p]
 * (fp32 add of the stored C value and the partial), written by the epilogue of
 * each tile; C holds this rank's own product as before.  Other backends,
 * bf16 C or COMPUTE_ONLY: EUNSUPPORTED; partials NULL: EINVAL. */
int sync_gemm_rs_reduce(sync_plan_t plan, const sync_copy_cfg* cfg, const void* a, const void* b, void* c,
                        const float* partials, void* staging, void* ws, void* compute, void* copy);

/* GEMM-AR share [SYN-S "Experiments", paper sec. 6.1 and Fig. 11: GEMM-AR;
 * a ring all-reduce is a reduce-scatter followed by an all-gather]: the
 * reduce-scatter half exactly as sync_gemm_rs_reduce (EPILOGUE backend, fp32
 * C; C, partials and staging as there), and in the same launch the
 * all-gather half: cfg->copy_cus CUs set aside for it from the start (0, or a
 * multiple of the XCD count up to half the CUs), and every compute
 * workgroup joins it once its tiles are stored:
 *   reduced_peer fp32 [m][n]: the fully reduced rows the peers send back in
 *                the all-gather, at their natural rows (read-only; the rows of
 *                this rank's own chunks are not read);
 *   out          fp32 [m][n]: the all-reduced result: this rank's own chunks
 *                from their staging slots (own tile + partials), every other
 *                chunk from reduced_peer.
 * The all-gather takes the chunks in ring order (this rank's own first, then
 * shard (rank - ring_dir k) mod world at step k), and sub-chunk q of every
 * shard waits in-kernel until this rank's own sub-chunk q is done, as the
 * all-gather of a sub-chunk follows its reduce-scatter on every rank. */
int sync_gemm_ar(sync_plan_t plan, const sync_copy_cfg* cfg, const void* a, const void* b, void* c,
                 const float* partials, const float* reduced_peer, float* out, void* staging, void* ws,
                 void* compute, void* copy);

/* Kernel-level overlap baseline of a GEMM plan [SYN-S "Key observations",
 * observation 1, Fig. 2(a)-(b); SYN-R Fig. 2 caption: the operator split into
 * per-chunk kernels whose communication overlaps through streams, which the
 * fused kernel is claimed to beat].  No fusion: for each chunk in the plan's
 * order,
 *   AG plan: a runtime copy of the chunk's rows from a_peer into a on `copy`
 *            (resident chunks are not copied), an event, and on `compute`
 *            after it a GEMM launch over those rows of a (every tile in
 *            place, tiles in row-major order);
 *   RS plan: a GEMM launch over the chunk's rows on `compute`, an event, and
 *            on `copy` after it a runtime copy of those rows of c into send
 *            slot p of `staging` (as sync_gemm_rs packs it); a_peer unused.
 * Then `compute` waits for `copy`, so the call is complete when `compute` is.
 * The GEMM kernel and its per-tile K order are those of the fused calls, so
 * the result is bitwise the same.  cfg: NULL or backend CU (runtime copies
 * on blit kernels) or SDMA (copies on the engines), no flags.  `copy` must
 * be a stream other than `compute`; ws as for the other calls.  Operands as
 * in sync_ag_gemm (a = a_local) or sync_gemm_rs. */
int sync_gemm_split(sync_plan_t plan, const sync_copy_cfg* cfg, const void* a_peer, void* a, const void* b,
                    void* c, int32_t c_dtype, void* staging, void* ws, void* compute, void* copy);

/* Ring-attention local step [SYN-S "Experiments", paper sec. 6.1 and Fig. 9:
 * RingAttention].  KV blocks (chunks of K and V token rows) are staged from
 * k_peer/v_peer into k_local/v_local in arrival order; each (query tile, head)
 * work item folds every block, in arrival order, into an fp32 online-softmax
 * state (m, l, O).
 *   q bf16 [m][heads_q][k]; k_*, v_* bf16 [world*n][heads_kv][k];
 *   o fp32 [m][heads_q][k]; m_state, l_state fp32 [heads_q][m];
 *   lse fp32 [heads_q][m] or NULL (written when FINALIZE).
 *   m_state is in natural-log units (max of scale * q.k); l_state is the sum
 *   of exp(score - m); o holds the unnormalised sum unless FINALIZE.  The
 *   probabilities multiplying V are rounded to bf16 (l sums them unrounded).
 *   flags: SYNC_ATTN_INIT starts from m=-inf, l=0, O=0 (else reads the
 *   state); SYNC_ATTN_FINALIZE writes O/l to o and m + ln l to lse (and the
 *   final m, l to the state).  Non-causal, no masking; scale > 0.
 * Kernel constraints (else EUNSUPPORTED): k (head dim) == 128;
 *   heads_q / heads_kv is 1, 2 or a multiple of 4.  The kernel groups the query
 *   heads of one KV head into its work items, so tile_m / tile_order of the
 *   plan do not change the result (every item needs every block). */
enum { SYNC_ATTN_INIT = 1, SYNC_ATTN_FINALIZE = 2 };
int sync_ring_attn_step(sync_plan_t plan, const sync_copy_cfg* cfg, const void* q,
                        const void* k_peer, const void* v_peer, void* k_local, void* v_local,
                        float* o, float* m_state, float* l_state, float* lse, float scale,
                        int32_t flags, void* ws, void* compute, void* copy);

/* Head-parallel attention share [SYN-S "Experiments", paper sec. 6.1 and
 * Fig. 9: head-parallel and sequence-parallel attention among the evaluated
 * operators; the pages give no scheme, the one used is DeepSpeed-Ulysses', in
 * SYN-R's references].  Before attention every rank holds a sequence shard of
 * n tokens of all heads; an all-to-all turns it into a head shard: this rank
 * receives, from every peer w, the n tokens [w*n, (w+1)*n) of its own head
 * group.  This call is that receive side fused with the attention over all
 * world*n tokens of the group: Q, K and V chunks (token blocks, in the plan's
 * arrival order) are staged from q_peer/k_peer/v_peer into q/k/v, and each
 * (query block, head group) work item starts once the chunks holding its
 * queries are in place, then folds the KV chunks in as they land, with the
 * same fp32 online softmax as sync_ring_attn_step.
 *   plan: op HEAD_ATTN, m = world*n, heads_q / heads_kv = this rank's group.
 *   q_* bf16 [world*n][heads_q][k]; k_*, v_* bf16 [world*n][heads_kv][k];
 *   the *_peer tensors hold at rows [w*n, (w+1)*n) what peer w sends (on one
 *   GPU: device buffers standing for the peers'); q, k, v are filled with
 *   every non-resident chunk's rows (the resident one, this rank's own
 *   block, must be in place already).
 *   o fp32 [world*n][heads_q][k] = softmax(scale q.k^T) v per head (query
 *   head h reads KV head h / (heads_q / heads_kv)); lse fp32 [heads_q][world*n]
 *   (natural log of the softmax denominator) or NULL.
 * Kernel constraints (else EUNSUPPORTED): k == 128; heads_q / heads_kv is 1,
 *   2 or a multiple of 4; tile_m == sync_attn_query_block(heads_q, heads_kv)
 *   (the query rows of one kernel work item); the plan's tile order is the
 *   order work items are taken in.  cfg as for sync_ring_attn_step (backends
 *   CU, COLOCATED, SDMA or PRESET; COPY_ONLY, COMPUTE_ONLY, TIMED, WITHHOLD).
 *   A work item whose chunks never arrive leaves its outputs untouched and
 *   the call returns ETIMEOUT. */
int sync_head_attn(sync_plan_t plan, const sync_copy_cfg* cfg, const void* q_peer, const void* k_peer,
                   const void* v_peer, void* q, void* k, void* v, float* o, float* lse, float scale, void* ws,
                   void* compute, void* copy);

/* Query rows of one work item of the attention kernel for this head
 * grouping (the tile_m a HEAD_ATTN plan must use); 0 if the grouping has no
 * kernel variant.  Needs no device. */
int32_t sync_attn_query_block(int32_t heads_q, int32_t heads_kv);

/* ---- autotuner ------------------------------------------------------------ */
/* Picks the fastest overlapped configuration of a GEMM call (AG or RS) by
 * running it over split factor (chunk size), tile shape, tile order and copy
 * agent (backend, copy-CU count, ...) [SYN-S "Core method": plans are tuned
 * per workload, and the pages leave the tuning cost out].
 * Every candidate in the cross product of the space's lists is planned from
 * `base` (its split, tile_m/tile_n, tile_order replaced), run `warmup` times
 * and then timed over `iters` calls with device events on `bufs->stream`.
 * Candidates the kernels do not support, or whose calls time out (each call
 * is bounded by timeout_ns, default 100 ms here), are skipped.  The copy side
 * of a candidate is either each entry of `agents` (copy configurations: SDMA
 * with its engine count in copy_teams, CU with copy_cus / copy_teams /
 * copy_kslices / copy_link_gbps, COLOCATED, or EPILOGUE for GEMM-RS; no flags
 * or host gates), or, with n_agents = 0, the CU backend at each count of the
 * copy_cus list.  Candidates an agent does not support (e.g. EPILOGUE for
 * AG) are skipped.
 * Results are cached per (device, HIP runtime version, op, shape, base fields, c_dtype, space) for
 * the life of the process, and in the text file named by the environment
 * variable SYNC_TUNE_CACHE when it is set (read on first use, appended after
 * each tuning); a cached result returns at once with candidates_run = 0
 * unless `force` is set.  The caller's buffers are overwritten by the runs
 * (c, staging, the non-resident rows of a_local, the workspace). */
typedef struct {
  const int32_t* splits;    int32_t n_splits;   /* split factors */
  const int32_t* tiles;     int32_t n_tiles;    /* n_tiles pairs (tile_m, tile_n) */
  const int32_t* orders;    int32_t n_orders;   /* SYNC_ORDER_* */
  const int32_t* copy_cus;  int32_t n_copy_cus; /* CU backend copy-CU counts */
  int32_t warmup, iters;   /* per candidate; 0 = 3 and 10 */
  uint64_t timeout_ns;     /* per-call device wait bound while tuning; 0 = 100 ms */
  int32_t force;           /* 1 = ignore cached results */
  int32_t reserved;        /* must be zero */
  const sync_copy_cfg* agents; int32_t n_agents; /* copy agents to try; 0 = the copy_cus list */
} sync_tune_space;

typedef struct {
  const void* a_peer;  /* AG: bf16 [m][k] peer region; RS: unused */
  void* a;             /* AG: a_local (resident shard filled); RS: a */
  const void* b;
  void* c;
  void* staging;       /* RS only */
  int32_t c_dtype;     /* SYNC_DTYPE_* */
  void* ws;            /* >= sync_tune_workspace_size() bytes, 256-byte aligned */
  void* stream;        /* compute stream */
} sync_tune_buffers;

typedef struct {
  int32_t split, tile_m, tile_n, tile_order, copy_cus;
  float best_ms;            /* mean call time of the winner */
  int32_t candidates_run;   /* 0 when served from the cache */
  int32_t candidates_skipped;
  int32_t backend;          /* SYNC_COPY_* of the winner */
  int32_t agent;            /* index of the winner in agents, -1 when from the copy_cus list */
  int32_t from_cache;       /* 1 when served from the cache (in-process or file) */
  float call_wall_ms;       /* host wall time of this sync_autotune call */
  float search_wall_ms;     /* host wall time the search that produced the result took (kept in the cache) */
} sync_tune_result;

/* Workspace bytes that fit every candidate of the space (0 on bad input). */
size_t sync_tune_workspace_size(const sync_plan_desc* base, const sync_tune_space* space);

int sync_autotune(const sync_plan_desc* base, const sync_tune_space* space, const sync_tune_buffers* bufs,
                  sync_tune_result* out);

/* Drops the in-process cache of tuning results (the cache file, if any, is
 * kept and read again on the next sync_autotune). */
void sync_tune_forget(void);

/* Durations of the most recent SYNC_RUN_TIMED calls on the current device
 * (a ring of 1024), oldest first; waits for those events.  kernel_ms is the
 * call's kernel launch (GEMM or attention; with the CU backend its copy
 * workgroups are part of it) from just before the launch to just after it, on
 * the stream it runs on (SDMA: from before the gate kernel to after the
 * compute or join kernel); copy_ms spans the copies (SDMA: the same span as
 * kernel_ms; 0 if none).  Reading
 * empties the ring.  *count = records written to out (<= max). */
typedef struct {
  float kernel_ms;
  float copy_ms;
} sync_timing;

int sync_read_timings(int32_t max, sync_timing* out, int32_t* count);

/* ---- device facts and housekeeping -------------------------------------- */
typedef struct {
  int32_t device;        /* HIP device ordinal (current device) */
  int32_t num_cus;       /* multiprocessor count */
  int32_t num_xcds;      /* XCDs (8 on MI355X) */
  int32_t clock_khz;     /* peak shader clock */
  int64_t wall_clock_khz;/* device wall clock used for wait time limits */
  char arch[64];         /* gcnArchName */
} sync_device_info;

int sync_get_device_info(sync_device_info* out);

/* Thread-local message for the last failing call on this thread. */
const char* sync_last_error(void);

/* Destroys the library's streams, events and SDMA signals on every device
 * (first waiting, bounded, for queued SDMA copies).  Only when no call is in
 * flight; the next call re-creates what it needs. */
void sync_shutdown(void);

#ifdef __cplusplus
}
#endif
#endif /* SYNC_OVERLAP_H */
