/*
 * bpe.h -- C ABI of the MI355X byte-level BPE library (libbpe.so).
 *
 * The operation (sources named by page title and section):
 *  - "Tokenization LLM: details of building an inference engine in C++"
 *    (glitch4techs.com), sections "Technical analysis" (a fixed pattern splits
 *    text into words, numbers, punctuation and whitespace, each piece handled
 *    on its own), "Byte-level encoding" (text is UTF-8 bytes), "BPE algorithm"
 *    (repeatedly merge the adjacent pair with the lowest rank until no ranked
 *    pair is left) and "Vocabulary lookup" (merged symbols become integer IDs).
 *  - "Characters, bytes and subwords" (tokenwerk.deckle.io), section "BPE step
 *    by step": a merge acts on the current sequence from the left without
 *    overlap, so [a,a,a] with (a,a) gives [aa,a]; section "Check the round
 *    trip first": decode(encode(x)) == x.
 *  - "Hugging Face Tokenizers v1: encoding up to 30x faster" (dothoosh.com),
 *    sections "How v1 works" (a merge never crosses a pre-token boundary),
 *    "Merge-loop rewrite" (caller-managed scratch, batches of pre-tokens) and
 *    "Road to 1.0.0" (batch encode/decode on the GPU with the vocabulary
 *    uploaded once, output positions computed in parallel, bytes gathered on
 *    the device; IDs-only output).
 *
 * Fixed readings of what the pages leave open:
 *  - Byte classes: L = A-Z, a-z and every byte >= 0x80; D = 0-9;
 *    W = 0x09-0x0D and 0x20; P = every other byte.
 *  - Split: the leftmost-first alternation of greedy runs
 *    ` ?L+ | D+ | P+ | W+` (only the space 0x20 may lead a letter run).
 *    Every document start is a pre-token start.
 *  - One merge step takes the smallest rank r* among all adjacent pairs of the
 *    pre-token and replaces every occurrence of pair(r*) in one left-to-right,
 *    non-overlapping pass; steps repeat until no adjacent pair is ranked.
 *  - Bytes are symbols 0..255; the merge of rank r creates symbol 256 + r.
 *    The output ID of a symbol is the symbol, or id_map[symbol].
 *
 * Conventions for every call:
 *  - Arguments named d_* are device pointers on the device that was current
 *    when the model was loaded; every other pointer is host memory.
 *  - Work is enqueued on `hip_stream` (a hipStream_t, or NULL for the null
 *    stream).  Encode and decode never synchronize the host; they return as
 *    soon as their kernels are queued.
 *  - Host-checkable problems return a negative BPE_E* code and enqueue
 *    nothing.  Problems only the device can see are reported in *d_status (an
 *    int32 in device memory that the call first clears) as BPE_STATUS_* bits;
 *    read it after synchronizing the stream.  When *d_status != 0 the outputs
 *    are not valid.
 *  - The caller owns all device buffers, including the workspace, which must
 *    not be shared by calls that may run at the same time.  A model is
 *    read-only after loading and may be used from several streams at once.
 */
#ifndef BPE_H
#define BPE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
#define BPE_OK 0
#define BPE_EINVAL (-1)      /* null pointer, negative size, unsupported size, wrong device */
#define BPE_EMERGES (-2)     /* merge table: repeated pair, operand out of range, or a cycle */
#define BPE_EIDMAP (-3)      /* id_map: negative, repeated, or above BPE_MAX_ID */
#define BPE_EWORKSPACE (-4)  /* workspace_bytes below what the *_workspace_bytes call gives */
#define BPE_EHIP (-5)        /* a HIP runtime call failed */
#define BPE_ENOMEM (-6)      /* host or device allocation failed while loading */
#define BPE_ENOTSUP (-7)     /* decode: this table's byte expansions exceed BPE_MAX_EXPANSION */
#define BPE_EFORMAT (-8)     /* text form: malformed line, JSON or UTF-8, or a character no byte prints as */
#define BPE_ESCRATCH (-9)    /* bpe_encode_batch_noalloc: the input needs more than BPE_NOALLOC_SCRATCH_BYTES */

/* bits of *d_status */
#define BPE_STATUS_BAD_DOC_OFFSETS 1u   /* encode: offsets not 0 = d[0] <= ... <= d[n_docs] = n_bytes */
#define BPE_STATUS_IDS_CAPACITY 2u      /* encode: more IDs than ids_capacity (extra IDs dropped) */
#define BPE_STATUS_BAD_ID 4u            /* decode: an ID that no symbol maps to */
#define BPE_STATUS_BYTES_CAPACITY 8u    /* decode: more bytes than bytes_capacity (extra dropped) */
#define BPE_STATUS_BAD_ID_OFFSETS 16u   /* decode: offsets not 0 = o[0] <= ... <= o[n_docs] = n_ids */

/* limits */
#define BPE_MAX_MERGES (1 << 20)               /* merges per table */
#define BPE_MAX_ID ((1 << 24) - 1)             /* largest value an id_map may hold */
#define BPE_MAX_EXPANSION ((int64_t)1 << 30)   /* total decoded bytes of all symbols, for decode */

typedef struct bpe_model bpe_model;

/*
 * Load a merge table ("merges.txt" of the C++ engine page, as integers).
 *  merges   host int32 [n_merges][2]: row r is the pair (left, right) whose
 *           merge has rank r and creates symbol 256 + r.  Operands are
 *           symbols in [0, 256 + n_merges).  Pairs must be distinct and no
 *           symbol may depend on itself through its operands.  Ranks need not
 *           follow creation order.  May be NULL when n_merges == 0.
 *  n_merges 0 <= n_merges <= BPE_MAX_MERGES.
 *  id_map   host int32 [256 + n_merges] or NULL (identity): the output ID of
 *           each symbol; values distinct, in [0, BPE_MAX_ID].
 *  out      receives the model; free it with bpe_free.
 * The tables are copied to the current device on hip_stream, and the call
 * waits for the copies.  Returns BPE_OK, BPE_EINVAL, BPE_EMERGES,
 * BPE_EIDMAP, BPE_ENOMEM or BPE_EHIP; *out is set only on success.
 */
int bpe_load_merges(const int32_t *merges, int64_t n_merges, const int32_t *id_map,
                    void *hip_stream, bpe_model **out);

/*
 * The text form of a table ("Tokenization LLM: details of building an
 * inference engine in C++", section "Byte-level encoding": every byte value
 * prints as one character, e.g. 0xF0 as U+00F0, so that merges and
 * vocabularies are stored as text; section "Vocabulary lookup": merged
 * symbols map to IDs through the vocabulary, where " world" is "Ġworld").
 * Printable map: bytes 0x21-0x7E, 0xA1-0xAC and 0xAE-0xFF print as the code
 * point of the same value, the other 68 bytes as U+0100, U+0101, ... in
 * increasing byte order (0x20 is U+0120 'Ġ').  Both calls run on the host
 * only; their results go to bpe_load_merges.
 *
 * Parse a merges file: UTF-8 text, one merge per line ("left right", one
 * space), in rank order, after an optional first line starting with
 * "#version"; empty lines are skipped and a line may end in a carriage
 * return (0x0D) before its line feed.  Each
 * operand is a byte or the text of an earlier line's result, and no two lines
 * may give the same bytes.
 *  merges_out  host int32 [max_merges][2]: row r receives line r's operands
 *              as symbols (bytes 0..255, line r' as 256 + r').
 *  n_merges    receives the number of merges.
 * Returns BPE_OK; BPE_EFORMAT (malformed line or UTF-8, or a character no
 * byte prints as); BPE_EMERGES (unknown operand, a repeated result, or more
 * than BPE_MAX_MERGES); BPE_EINVAL (null pointer, or more than max_merges).
 */
int bpe_parse_merges_text(const char *text, int64_t text_len, int32_t *merges_out,
                          int64_t max_merges, int64_t *n_merges);

/*
 * Parse a vocabulary: a JSON object from token text (in the printable map)
 * to integer ID, e.g. {"hello": 15339, "\u0120world": 1917}.  Keys with
 * characters outside the printable map name no symbol and are ignored (the
 * names of reserved IDs, for instance).
 *  merges      host int32 [n_merges][2], the table (as bpe_load_merges).
 *  id_map_out  host int32 [256 + n_merges]: receives each symbol's ID, the
 *              ID of the text of its bytes; ready for bpe_load_merges.
 * Returns BPE_OK; BPE_EFORMAT (malformed JSON); BPE_EMERGES (operand out of
 * range or a cycle); BPE_EIDMAP (a symbol's text missing, or its ID outside
 * [0, BPE_MAX_ID]); BPE_EINVAL (null pointer or bad size).
 */
int bpe_parse_vocab_json(const char *json, int64_t json_len, const int32_t *merges,
                         int64_t n_merges, int32_t *id_map_out);

/*
 * Train a merge table on the current device ("Characters, bytes and
 * subwords", section "BPE step by step": count the adjacent pairs, the most
 * frequent one merges into a new symbol (ties: the smallest IDs), replace its
 * occurrences, count again, until n_merges merges or no pair occurs twice;
 * "Hugging Face Tokenizers v1", section "How v1 works": merges stay inside
 * pre-tokens).  Readings: pairs are counted at every position, weighted by
 * the pre-token's frequency in the corpus; ties go to the smallest (left,
 * right); replacement is encoding's left-to-right pass without overlap.
 *  bytes, doc_off  host memory: the corpus as for bpe_encode_batch (offsets
 *                  that are not 0 = d[0] <= ... <= d[n_docs] = n_bytes give
 *                  BPE_EINVAL); n_bytes below 2^32, and the distinct
 *                  pre-tokens' bytes below 2^30, else BPE_EINVAL.
 *  merges_out      host int32 [n_merges][2]: merge r, rank order.
 *  counts_out      host int64 [n_merges] or NULL: each merge's pair count.
 *  n_made          receives the number of merges made (<= n_merges).
 * The distinct pre-tokens are collected on the host; the device counts the
 * pairs once, then keeps the counts up to date merge by merge (a merge
 * changes only the pre-tokens that hold its pair).  The call allocates its
 * own device memory, runs on hip_stream (and a stream of its own, ordered
 * after it) and waits for the result.  Returns BPE_OK, BPE_EINVAL,
 * BPE_ENOMEM or BPE_EHIP.
 */
int bpe_train(const uint8_t *bytes, int64_t n_bytes, const int64_t *doc_off, int64_t n_docs,
              int64_t n_merges, int32_t *merges_out, int64_t *counts_out, int64_t *n_made,
              void *hip_stream);

/* Release a model and its device tables (the caller makes sure no queued
 * work still uses it).  NULL is ignored. */
void bpe_free(bpe_model *model);

/* 256 + n_merges, or -1 for NULL. */
int64_t bpe_vocab_size(const bpe_model *model);

/* Largest token length in bytes (1 if there are no merges), or -1 for NULL or
 * when decode is unsupported for this table. */
int64_t bpe_max_token_bytes(const bpe_model *model);

/* Workspace bytes bpe_encode_batch needs for this input size (0 for
 * n_bytes <= 0): about 28.7 bytes per input byte plus 4 per document, since
 * every intermediate region is sized for the worst case of each 4 KiB chunk
 * (for example 7.5 GiB for a 256 MiB batch). */
size_t bpe_encode_workspace_bytes(const bpe_model *model, int64_t n_bytes, int64_t n_docs);

/*
 * Encode a batch of documents into token IDs.
 *  d_bytes       uint8 [n_bytes]: the documents back to back (UTF-8 or any
 *                bytes; no byte is special).
 *  d_doc_off     int64 [n_docs + 1]: document d is d_bytes[d_doc_off[d] ..
 *                d_doc_off[d+1]); must satisfy 0 = d_doc_off[0] <= ... <=
 *                d_doc_off[n_docs] = n_bytes, else BPE_STATUS_BAD_DOC_OFFSETS
 *                is set and the outputs are not valid (every write still stays
 *                inside the caller's buffers).  Empty documents are allowed.
 *  d_ids         int32 [ids_capacity]: receives the IDs of all documents in
 *                order.  The count never exceeds n_bytes, so ids_capacity >=
 *                n_bytes always suffices; with less, IDs at index >=
 *                ids_capacity are dropped and BPE_STATUS_IDS_CAPACITY is set.
 *  d_id_off      int64 [n_docs + 1]: receives the offsets of each document's
 *                IDs; d_id_off[n_docs] is the total ID count.
 *  d_workspace   device scratch of workspace_bytes >=
 *                bpe_encode_workspace_bytes(model, n_bytes, n_docs).
 *  d_status      int32 [1]: cleared, then receives BPE_STATUS_* bits.
 * Returns BPE_OK, BPE_EINVAL, BPE_EWORKSPACE or BPE_EHIP.
 */
int bpe_encode_batch(const bpe_model *model, const uint8_t *d_bytes, int64_t n_bytes,
                     const int64_t *d_doc_off, int64_t n_docs, int32_t *d_ids,
                     int64_t ids_capacity, int64_t *d_id_off, void *d_workspace,
                     size_t workspace_bytes, int32_t *d_status, void *hip_stream);

/*
 * Encode with no allocation and no caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace is a static device array of
 * BPE_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, which each GPU
 * holds from the first such call on it until the process ends; its device
 * address is looked up once per device, on that first call.  The call itself
 * allocates nothing (no hipMalloc, hipFree or allocating library routine, and
 * no stage-timing events).
 *  Arguments, outputs, status bits and the operation are bpe_encode_batch's,
 *  without d_workspace / workspace_bytes.
 *  Inputs whose bpe_encode_workspace_bytes(model, n_bytes, n_docs) exceeds
 *  BPE_NOALLOC_SCRATCH_BYTES are rejected with BPE_ESCRATCH before anything is
 *  queued.
 *  Every call on one GPU shares that GPU's array: calls that may overlap on one
 *  GPU (several streams or host threads) race and must be serialized by the
 *  caller.  The array keeps the last call's contents; the kernels clear what
 *  they need cleared themselves.
 * Returns BPE_OK, BPE_EINVAL, BPE_ESCRATCH or BPE_EHIP.
 */
#define BPE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int bpe_encode_batch_noalloc(const bpe_model *model, const uint8_t *d_bytes, int64_t n_bytes,
                             const int64_t *d_doc_off, int64_t n_docs, int32_t *d_ids,
                             int64_t ids_capacity, int64_t *d_id_off, int32_t *d_status,
                             void *hip_stream);

/*
 * Reserved IDs around each document: post-processing ("Characters, bytes and
 * subwords", section "Special tokens are their own IDs": IDs such as BOS and
 * EOS are reserved, inserted on purpose when data is prepared, and no text
 * can produce them; "Hugging Face Tokenizers v1", section "How v1 works": a
 * post-processing stage adds the special tokens a model expects).
 *
 * Workspace bytes bpe_encode_batch_special needs: the same as
 * bpe_encode_batch (0 for n_bytes <= 0).
 */
size_t bpe_encode_special_workspace_bytes(const bpe_model *model, int64_t n_bytes,
                                          int64_t n_docs);

/*
 * Encode as bpe_encode_batch, then put bos_id before and eos_id after each
 * document's IDs (also around an empty document).  Either may be -1 (none);
 * otherwise it must lie in [0, BPE_MAX_ID] and be no symbol's output ID
 * (with an id_map, no value of it; else not below 256 + n_merges), so that
 * no text yields it, else BPE_EINVAL.
 *  d_ids       receives document d's IDs as [bos] encode(d) [eos]; the count
 *              is at most n_bytes + n_docs * (number of reserved IDs given),
 *              and with less capacity the IDs past it are dropped and
 *              BPE_STATUS_IDS_CAPACITY is set.
 *  d_id_off    receives each document's offset, the reserved IDs included.
 * Other arguments, the workspace, the status bits and the return codes as
 * bpe_encode_batch.  The reserved IDs are written by the encode's own last
 * kernel: the call costs about what bpe_encode_batch does.
 */
int bpe_encode_batch_special(const bpe_model *model, const uint8_t *d_bytes, int64_t n_bytes,
                             const int64_t *d_doc_off, int64_t n_docs, int32_t bos_id,
                             int32_t eos_id, int32_t *d_ids, int64_t ids_capacity,
                             int64_t *d_id_off, void *d_workspace, size_t workspace_bytes,
                             int32_t *d_status, void *hip_stream);

/* Workspace bytes bpe_decode_batch needs (0 for n_ids <= 0). */
size_t bpe_decode_workspace_bytes(const bpe_model *model, int64_t n_ids, int64_t n_docs);

/*
 * Decode token IDs back to bytes (the inverse of encode, byte for byte).
 *  d_ids         int32 [n_ids]; an ID that is not the output ID of any symbol
 *                sets BPE_STATUS_BAD_ID (it contributes no bytes).
 *  d_id_off      int64 [n_docs + 1] with 0 = o[0] <= ... <= o[n_docs] = n_ids,
 *                else BPE_STATUS_BAD_ID_OFFSETS is set and the outputs are not
 *                valid (every write still stays inside the caller's buffers).
 *  d_bytes       uint8 [bytes_capacity]: receives the bytes of all documents;
 *                bytes past the capacity are dropped and
 *                BPE_STATUS_BYTES_CAPACITY is set.  n_ids * bpe_max_token_bytes
 *                always suffices.
 *  d_byte_off    int64 [n_docs + 1]: receives the byte offsets per document.
 * Returns BPE_OK, BPE_EINVAL, BPE_EWORKSPACE, BPE_ENOTSUP or BPE_EHIP.
 */
int bpe_decode_batch(const bpe_model *model, const int32_t *d_ids, int64_t n_ids,
                     const int64_t *d_id_off, int64_t n_docs, uint8_t *d_bytes,
                     int64_t bytes_capacity, int64_t *d_byte_off, void *d_workspace,
                     size_t workspace_bytes, int32_t *d_status, void *hip_stream);

/*
 * Decode as bpe_decode_batch, with the reserved IDs skip_a and skip_b (each
 * -1 for none, else a valid reserved ID as for bpe_encode_batch_special,
 * else BPE_EINVAL) decoding to no bytes instead of setting
 * BPE_STATUS_BAD_ID: the output of bpe_encode_batch_special decodes back to
 * the input bytes ("Special tokens are their own IDs": on output they may be
 * skipped).  Same workspace as bpe_decode_batch.
 */
int bpe_decode_batch_special(const bpe_model *model, const int32_t *d_ids, int64_t n_ids,
                             const int64_t *d_id_off, int64_t n_docs, int32_t skip_a,
                             int32_t skip_b, uint8_t *d_bytes, int64_t bytes_capacity,
                             int64_t *d_byte_off, void *d_workspace, size_t workspace_bytes,
                             int32_t *d_status, void *hip_stream);

/*
 * Stage timing, for benchmarks and profilers.  While it is enabled on a
 * model, each bpe_encode_batch / bpe_decode_batch call with input records a
 * HIP event on its stream before its first kernel and after each kernel
 * (event records only: the call still never synchronizes).  While enabled,
 * calls on the model must come from one host thread.
 *  bpe_stage_timing   enable (1) or disable (0); either way, events not yet
 *                     read are dropped.  Returns BPE_OK, BPE_EINVAL or BPE_EHIP.
 *  bpe_stage_count    number of kernels (stages) of op, or -1.
 *  bpe_stage_name     static name of a stage, or NULL.
 *  bpe_stage_times    waits for the recorded events of op, writes each
 *                     stage's total milliseconds over the calls since the
 *                     last read to ms[0 .. bpe_stage_count(op)), and the
 *                     number of those calls to *n_calls; then forgets them.
 *                     max_stages is the length of ms.  Returns BPE_OK,
 *                     BPE_EINVAL or BPE_EHIP.
 */
#define BPE_OP_ENCODE 0
#define BPE_OP_DECODE 1
int bpe_stage_timing(bpe_model *model, int enable);
int bpe_stage_count(int op);
const char *bpe_stage_name(int op, int stage);
int bpe_stage_times(bpe_model *model, int op, double *ms, int max_stages, int64_t *n_calls);

/* A static English description of a BPE_E* code. */
const char *bpe_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* BPE_H */
