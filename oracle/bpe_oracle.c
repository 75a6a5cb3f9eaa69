/*
 * bpe_oracle.c -- plain, slow, single-threaded CPU oracle for byte-level BPE.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library.  It shares no code,
 * header, table or helper with the GPU library under
 * byte_level_bpe_pretokenize_amd/, and neither side includes the other.
 *
 * Sources (the pages' titles; sections in parentheses):
 *  [P1] "Tokenization LLM: details of building an inference engine in C++"
 *       (glitch4techs.com): Technical analysis (regex split, 'Hello world!'),
 *       Byte-level encoding (UTF-8 bytes, byte->unicode map, 0xF0 -> U+00F0),
 *       BPE algorithm (ranked merge loop, lower rank merges first),
 *       Vocabulary lookup (merged symbols -> IDs).
 *  [P3] "Characters, bytes and subwords" (tokenwerk.deckle.io):
 *       Bytes as a robust foundation (256 byte tokens), BPE step by step
 *       (count adjacent pairs, most frequent wins, ties -> smallest IDs,
 *       left-to-right non-overlapping replacement, [a,a,a] -> [aa,a]),
 *       Check the round trip first (decode(encode(x)) == x).
 *  [P4] "Hugging Face Tokenizers v1: encoding up to 30x faster"
 *       (dothoosh.com): How v1 works (BPE definition, merges never cross a
 *       pre-token boundary), Benchmarks (FNV-1a over output IDs).
 *
 * Readings where the pages are silent:
 *  R1 byte classes: L = A-Z a-z and every byte >= 0x80; D = 0-9;
 *     W = 0x09-0x0D and 0x20; P = every other byte.
 *  R2 split: leftmost-first alternation of greedy runs ` ?L+ | D+ | P+ | W+`,
 *     the optional leading character being the space 0x20 only.
 *  R3 every document start is a pre-token start; empty documents give 0 IDs.
 *  R4 one merge step: take the smallest rank r* among adjacent pairs, then
 *     replace every occurrence of pair(r*) in one left-to-right,
 *     non-overlapping pass; repeat until no adjacent pair has a rank.
 *  R5 legal tables: unique pairs, operands < 256+R, acyclic operand graph.
 *  R6 bytes are symbols 0..255, rank r creates symbol 256+r; the output ID is
 *     the symbol, or id_map[symbol] when a map is given.
 *  R7 trainer: positional pair counts weighted by pre-token frequency; most
 *     frequent pair wins, ties to the smallest (left, right); replacement per
 *     R4; stop after N merges or when the best count is below 2.
 *  R8 byte->unicode: bytes 0x21-0x7E, 0xA1-0xAC, 0xAE-0xFF keep their code
 *     point; the other 68 bytes map in increasing order to U+0100..U+0143.
 *  R9 decode concatenates byte expansions and returns raw bytes.
 *  R12 checksum: 64-bit FNV-1a over the little-endian int32 ID stream.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORA_INF INT32_MAX

/* ------------------------------------------------------------------ R1 -- */
/* [P1] Technical analysis: the split separates words, numbers, punctuation
 * and whitespace.  The class table itself is reading R1. */
enum { CLS_L = 0, CLS_D = 1, CLS_W = 2, CLS_P = 3 };

int ora_byte_class(int b)
{
    if ((b >= 'A' && b <= 'Z') || (b >= 'a' && b <= 'z') || b >= 0x80)
        return CLS_L;
    if (b >= '0' && b <= '9')
        return CLS_D;
    if ((b >= 0x09 && b <= 0x0D) || b == 0x20)
        return CLS_W;
    return CLS_P;
}

/* ------------------------------------------------------------------ R2 -- */
/* Length of the pre-token that begins at s[i] (i < n), following the
 * alternation ` ?L+ | D+ | P+ | W+` tried left to right, each run greedy. */
static int64_t match_at(const uint8_t *s, int64_t n, int64_t i)
{
    int64_t j;
    /* alternative 1: optional space, then one or more letters */
    if (s[i] == 0x20 && i + 1 < n && ora_byte_class(s[i + 1]) == CLS_L) {
        j = i + 2;
        while (j < n && ora_byte_class(s[j]) == CLS_L) j++;
        return j - i;
    }
    /* alternatives 1 (no space), 2, 3, 4: a maximal run of s[i]'s class */
    int c = ora_byte_class(s[i]);
    j = i + 1;
    while (j < n && ora_byte_class(s[j]) == c) j++;
    return j - i;
}

/* Split one document; writes the start offset of every pre-token.
 * Returns the number of pre-tokens (<= n). */
int64_t ora_split(const uint8_t *s, int64_t n, int64_t *starts)
{
    int64_t k = 0, i = 0;
    while (i < n) {
        starts[k++] = i;
        i += match_at(s, n, i);
    }
    return k;
}

/* ------------------------------------------------------------------ R8 -- */
/* [P1] Byte-level encoding: every byte value gets a printable code point;
 * 0xF0 maps to U+00F0.  The construction is reading R8. */
int ora_byte_to_unicode(int b)
{
    if ((b >= 0x21 && b <= 0x7E) || (b >= 0xA1 && b <= 0xAC) || (b >= 0xAE && b <= 0xFF))
        return b;
    int k = 0;
    for (int x = 0; x < b; x++) {
        int keeps = (x >= 0x21 && x <= 0x7E) || (x >= 0xA1 && x <= 0xAC) || (x >= 0xAE && x <= 0xFF);
        if (!keeps) k++;
    }
    return 0x100 + k;
}

/* UTF-8 encoding of one code point ([P1] Byte-level encoding, [P3] Bytes).
 * Returns the byte count (1..4), or 0 for a value outside U+0000..U+10FFFF
 * or in the surrogate range. */
int ora_utf8_encode(uint32_t cp, uint8_t *out)
{
    if (cp < 0x80) { out[0] = (uint8_t)cp; return 1; }
    if (cp < 0x800) {
        out[0] = (uint8_t)(0xC0 | (cp >> 6));
        out[1] = (uint8_t)(0x80 | (cp & 0x3F));
        return 2;
    }
    if (cp >= 0xD800 && cp <= 0xDFFF) return 0;
    if (cp < 0x10000) {
        out[0] = (uint8_t)(0xE0 | (cp >> 12));
        out[1] = (uint8_t)(0x80 | ((cp >> 6) & 0x3F));
        out[2] = (uint8_t)(0x80 | (cp & 0x3F));
        return 3;
    }
    if (cp <= 0x10FFFF) {
        out[0] = (uint8_t)(0xF0 | (cp >> 18));
        out[1] = (uint8_t)(0x80 | ((cp >> 12) & 0x3F));
        out[2] = (uint8_t)(0x80 | ((cp >> 6) & 0x3F));
        out[3] = (uint8_t)(0x80 | (cp & 0x3F));
        return 4;
    }
    return 0;
}

/* ----------------------------------------------------------------- R12 -- */
/* [P4] Benchmarks: the FNV-1a hash of the output IDs must match the
 * baseline's.  64-bit FNV-1a (offset basis 0xcbf29ce484222325, prime
 * 0x100000001b3), applied to a byte buffer. */
uint64_t ora_fnv1a64(const uint8_t *p, int64_t n)
{
    uint64_t h = 0xcbf29ce484222325ull;
    for (int64_t i = 0; i < n; i++) {
        h ^= p[i];
        h *= 0x100000001b3ull;
    }
    return h;
}

/* ----------------------------------------------------------- merge table -- */
/* [P1] BPE algorithm / Vocabulary lookup: a dictionary from a pair of units
 * to its rank; [P3] persist bytes and merges, merge order is part of the
 * encoder.  Readings R5, R6. */
typedef struct {
    uint64_t key;   /* (left << 32) | right */
    int32_t rank;
} PairRank;

typedef struct {
    int64_t R;
    int32_t *left, *right;   /* [R] */
    PairRank *sorted;        /* [R], sorted by key: lookup by binary search */
    int32_t *id_map;         /* NULL or [256+R] */
    PairRank *inv;           /* NULL or [256+R] (key = id, rank = symbol), sorted */
} OraTable;

static int cmp_pair(const void *a, const void *b)
{
    uint64_t x = ((const PairRank *)a)->key, y = ((const PairRank *)b)->key;
    return x < y ? -1 : x > y;
}

static uint64_t pkey(int32_t l, int32_t r)
{
    return ((uint64_t)(uint32_t)l << 32) | (uint32_t)r;
}

/* rank of pair (l, r) or ORA_INF */
static int32_t ora_rank(const OraTable *t, int32_t l, int32_t r)
{
    PairRank q = {pkey(l, r), 0};
    const PairRank *f = (const PairRank *)bsearch(&q, t->sorted, (size_t)t->R, sizeof(PairRank), cmp_pair);
    return f ? f->rank : ORA_INF;
}

/* Error codes of the oracle's table check (R5). */
#define ORA_OK 0
#define ORA_EINVAL -1
#define ORA_EDUP -2
#define ORA_ERANGE -3
#define ORA_ECYCLE -4
#define ORA_EIDMAP -5

/* R5: returns ORA_OK or the first problem found. */
int ora_validate(const int32_t *merges, int64_t R, const int32_t *id_map)
{
    if (R < 0 || (R > 0 && !merges)) return ORA_EINVAL;
    int64_t V = 256 + R;
    for (int64_t r = 0; r < R; r++)
        for (int k = 0; k < 2; k++)
            if (merges[2 * r + k] < 0 || merges[2 * r + k] >= V) return ORA_ERANGE;
    PairRank *s = (PairRank *)malloc(sizeof(PairRank) * (size_t)(R ? R : 1));
    for (int64_t r = 0; r < R; r++) { s[r].key = pkey(merges[2 * r], merges[2 * r + 1]); s[r].rank = (int32_t)r; }
    qsort(s, (size_t)R, sizeof(PairRank), cmp_pair);
    for (int64_t r = 1; r < R; r++)
        if (s[r].key == s[r - 1].key) { free(s); return ORA_EDUP; }
    free(s);
    /* acyclic: depth-first search from every merged symbol over its two
     * operands, colours 0 = unseen, 1 = on the stack, 2 = done */
    uint8_t *colour = (uint8_t *)calloc((size_t)V, 1);
    int64_t *stack = (int64_t *)malloc(sizeof(int64_t) * (size_t)(3 * V + 4));
    int rc = ORA_OK;
    for (int64_t root = 256; root < V && rc == ORA_OK; root++) {
        if (colour[root]) continue;
        int64_t sp = 0;
        stack[sp++] = root;       /* entry: symbol, >= 0 means "enter" */
        while (sp > 0 && rc == ORA_OK) {
            int64_t v = stack[--sp];
            if (v < 0) { colour[-v - 1] = 2; continue; }   /* exit marker */
            if (colour[v] == 2) continue;
            if (colour[v] == 1) continue;
            colour[v] = 1;
            stack[sp++] = -v - 1;
            if (v >= 256) {
                for (int k = 0; k < 2; k++) {
                    int64_t u = merges[2 * (v - 256) + k];
                    if (colour[u] == 1) { rc = ORA_ECYCLE; break; }
                    if (colour[u] == 0) stack[sp++] = u;
                }
            }
        }
    }
    free(stack);
    free(colour);
    if (rc != ORA_OK) return rc;
    if (id_map) {
        PairRank *m = (PairRank *)malloc(sizeof(PairRank) * (size_t)V);
        for (int64_t i = 0; i < V; i++) {
            if (id_map[i] < 0) { free(m); return ORA_EIDMAP; }
            m[i].key = (uint64_t)id_map[i];
            m[i].rank = (int32_t)i;
        }
        qsort(m, (size_t)V, sizeof(PairRank), cmp_pair);
        for (int64_t i = 1; i < V; i++)
            if (m[i].key == m[i - 1].key) { free(m); return ORA_EIDMAP; }
        free(m);
    }
    return ORA_OK;
}

void *ora_table_new(const int32_t *merges, int64_t R, const int32_t *id_map)
{
    if (ora_validate(merges, R, id_map) != ORA_OK) return NULL;
    OraTable *t = (OraTable *)calloc(1, sizeof(OraTable));
    t->R = R;
    size_t nr = (size_t)(R ? R : 1);
    t->left = (int32_t *)malloc(sizeof(int32_t) * nr);
    t->right = (int32_t *)malloc(sizeof(int32_t) * nr);
    t->sorted = (PairRank *)malloc(sizeof(PairRank) * nr);
    for (int64_t r = 0; r < R; r++) {
        t->left[r] = merges[2 * r];
        t->right[r] = merges[2 * r + 1];
        t->sorted[r].key = pkey(merges[2 * r], merges[2 * r + 1]);
        t->sorted[r].rank = (int32_t)r;
    }
    qsort(t->sorted, (size_t)R, sizeof(PairRank), cmp_pair);
    if (id_map) {
        int64_t V = 256 + R;
        t->id_map = (int32_t *)malloc(sizeof(int32_t) * (size_t)V);
        memcpy(t->id_map, id_map, sizeof(int32_t) * (size_t)V);
        t->inv = (PairRank *)malloc(sizeof(PairRank) * (size_t)V);
        for (int64_t i = 0; i < V; i++) { t->inv[i].key = (uint64_t)id_map[i]; t->inv[i].rank = (int32_t)i; }
        qsort(t->inv, (size_t)V, sizeof(PairRank), cmp_pair);
    }
    return t;
}

void ora_table_free(void *h)
{
    OraTable *t = (OraTable *)h;
    if (!t) return;
    free(t->left); free(t->right); free(t->sorted); free(t->id_map); free(t->inv);
    free(t);
}

/* ------------------------------------------------------------------ R4 -- */
/* [P1] BPE algorithm: split the pre-token into single byte units, look up
 * every adjacent pair, merge the pair with the lowest rank, repeat until no
 * valid merge remains.  [P3] BPE step by step: a merge acts on the current
 * sequence from the left without overlap.  Reading R4 makes one step replace
 * every occurrence of the chosen pair.  `sym` holds n symbols on entry and the
 * result on return; `tmp` has room for n symbols.  Returns the new length. */
static int64_t encode_symbols(const OraTable *t, int32_t *sym, int64_t n, int32_t *tmp)
{
    for (;;) {
        int32_t best = ORA_INF;
        for (int64_t i = 0; i + 1 < n; i++) {
            int32_t r = ora_rank(t, sym[i], sym[i + 1]);
            if (r < best) best = r;
        }
        if (best == ORA_INF) return n;
        int32_t L = t->left[best], Rt = t->right[best], z = 256 + best;
        int64_t o = 0, i = 0;
        while (i < n) {
            if (i + 1 < n && sym[i] == L && sym[i + 1] == Rt) {
                tmp[o++] = z;
                i += 2;
            } else {
                tmp[o++] = sym[i];
                i += 1;
            }
        }
        memcpy(sym, tmp, sizeof(int32_t) * (size_t)o);
        n = o;
    }
}

/* Encode one pre-token (bytes) into symbols; returns the symbol count. */
int64_t ora_encode_word(const void *h, const uint8_t *w, int64_t n, int32_t *out)
{
    const OraTable *t = (const OraTable *)h;
    int32_t *tmp = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n ? n : 1));
    for (int64_t i = 0; i < n; i++) out[i] = w[i];
    int64_t m = encode_symbols(t, out, n, tmp);
    free(tmp);
    return m;
}

/* [P1] Vocabulary lookup (reading R6): the output ID of a symbol. */
static int32_t symbol_id(const OraTable *t, int32_t s)
{
    return t->id_map ? t->id_map[s] : s;
}

/* Encode a batch of documents.  data[doc_off[d] .. doc_off[d+1]) is document
 * d.  Writes IDs in document order and id_off[0..n_docs].  Returns the total
 * ID count, or -1 if ids_cap is too small, or -2 for bad offsets. */
int64_t ora_encode_batch(const void *h, const uint8_t *data, int64_t n_bytes,
                         const int64_t *doc_off, int64_t n_docs,
                         int32_t *ids, int64_t ids_cap, int64_t *id_off)
{
    const OraTable *t = (const OraTable *)h;
    if (n_docs < 0 || doc_off[0] != 0 || doc_off[n_docs] != n_bytes) return -2;
    for (int64_t d = 0; d < n_docs; d++)
        if (doc_off[d + 1] < doc_off[d]) return -2;
    int64_t maxlen = 1;
    for (int64_t d = 0; d < n_docs; d++)
        if (doc_off[d + 1] - doc_off[d] > maxlen) maxlen = doc_off[d + 1] - doc_off[d];
    int64_t *starts = (int64_t *)malloc(sizeof(int64_t) * (size_t)(maxlen + 1));
    int32_t *sym = (int32_t *)malloc(sizeof(int32_t) * (size_t)maxlen);
    int32_t *tmp = (int32_t *)malloc(sizeof(int32_t) * (size_t)maxlen);
    int64_t T = 0;
    int64_t rc = 0;
    for (int64_t d = 0; d < n_docs && rc == 0; d++) {
        id_off[d] = T;
        const uint8_t *doc = data + doc_off[d];
        int64_t n = doc_off[d + 1] - doc_off[d];
        int64_t P = ora_split(doc, n, starts);
        starts[P] = n;
        for (int64_t k = 0; k < P; k++) {
            int64_t len = starts[k + 1] - starts[k];
            for (int64_t i = 0; i < len; i++) sym[i] = doc[starts[k] + i];
            int64_t m = encode_symbols(t, sym, len, tmp);
            if (T + m > ids_cap) { rc = -1; break; }
            for (int64_t i = 0; i < m; i++) ids[T + i] = symbol_id(t, sym[i]);
            T += m;
        }
    }
    if (rc == 0) id_off[n_docs] = T;
    free(starts); free(sym); free(tmp);
    return rc ? rc : T;
}

/* ------------------------------------------------------------------ R9 -- */
/* [P3] Check the round trip first: decoding concatenates what each token
 * stands for.  expansion(b) = [b] for a byte; expansion(256+r) =
 * expansion(left_r) followed by expansion(right_r).  Writes the bytes of
 * symbol s at out (if out != NULL) and returns their count; -1 if the byte
 * count would pass cap. */
static int64_t expand_symbol(const OraTable *t, int32_t s, uint8_t *out, int64_t cap,
                             int32_t *stack, int64_t stack_cap)
{
    int64_t sp = 0, n = 0;
    stack[sp++] = s;
    while (sp > 0) {
        int32_t v = stack[--sp];
        if (v < 256) {
            if (n >= cap) return -1;
            if (out) out[n] = (uint8_t)v;
            n++;
        } else {
            if (sp + 2 > stack_cap) return -1;
            stack[sp++] = t->right[v - 256];   /* pushed first, popped last */
            stack[sp++] = t->left[v - 256];
        }
    }
    return n;
}

/* symbol of an output ID, or -1 */
static int32_t id_symbol(const OraTable *t, int32_t id)
{
    if (!t->id_map) return (id >= 0 && id < 256 + t->R) ? id : -1;
    PairRank q = {(uint64_t)(uint32_t)id, 0};
    if (id < 0) return -1;
    const PairRank *f = (const PairRank *)bsearch(&q, t->inv, (size_t)(256 + t->R), sizeof(PairRank), cmp_pair);
    return f ? f->rank : -1;
}

/* Decode a batch.  Returns the total byte count, -1 if out_cap is too small,
 * -2 for bad offsets, -3 for an ID with no symbol. */
int64_t ora_decode_batch(const void *h, const int32_t *ids, int64_t n_ids,
                         const int64_t *id_off, int64_t n_docs,
                         uint8_t *out, int64_t out_cap, int64_t *byte_off)
{
    const OraTable *t = (const OraTable *)h;
    if (n_docs < 0 || id_off[0] != 0 || id_off[n_docs] != n_ids) return -2;
    for (int64_t d = 0; d < n_docs; d++)
        if (id_off[d + 1] < id_off[d]) return -2;
    int64_t stack_cap = 2 * (256 + t->R) + 4;
    int32_t *stack = (int32_t *)malloc(sizeof(int32_t) * (size_t)stack_cap);
    int64_t n = 0, rc = 0;
    for (int64_t d = 0; d < n_docs && rc == 0; d++) {
        byte_off[d] = n;
        for (int64_t k = id_off[d]; k < id_off[d + 1]; k++) {
            int32_t s = id_symbol(t, ids[k]);
            if (s < 0) { rc = -3; break; }
            int64_t m = expand_symbol(t, s, out ? out + n : NULL, out_cap - n, stack, stack_cap);
            if (m < 0) { rc = -1; break; }
            n += m;
        }
    }
    if (rc == 0) byte_off[n_docs] = n;
    free(stack);
    return rc ? rc : n;
}

/* ------------------------------------------------------------------ R7 -- */
/* [P3] BPE step by step: start from bytes, count adjacent token pairs over
 * the training corpus, take the most frequent pair (ties: the one with the
 * smallest IDs), give it a new ID, replace its occurrences, count again; stop
 * after the requested number of merges or when no pair is frequent enough.
 *
 * Distinct pre-tokens and their frequencies come first ([P4] How v1 works:
 * a merge never crosses a pre-token boundary). */

typedef struct {
    int32_t *sym;
    int64_t n;
    int64_t freq;
} Word;

typedef struct {
    const uint8_t *p;
    int64_t n;
    int64_t count;
    int used;
} WordSlot;

static uint64_t hash_bytes(const uint8_t *p, int64_t n)
{
    return ora_fnv1a64(p, n) * 0x9E3779B97F4A7C15ull;
}

/* Distinct pre-tokens of the corpus with their counts (open addressing,
 * doubled when half full). */
static void word_insert(WordSlot *tab, int64_t cap, const uint8_t *w, int64_t len, int64_t count,
                        int64_t *distinct)
{
    int64_t i = (int64_t)(hash_bytes(w, len) & (uint64_t)(cap - 1));
    for (;;) {
        if (!tab[i].used) {
            tab[i].used = 1; tab[i].p = w; tab[i].n = len; tab[i].count = count;
            (*distinct)++;
            return;
        }
        if (tab[i].n == len && memcmp(tab[i].p, w, (size_t)len) == 0) {
            tab[i].count += count;
            return;
        }
        i = (i + 1) & (cap - 1);
    }
}

static Word *collect_words(const uint8_t *data, int64_t n_bytes, const int64_t *doc_off,
                           int64_t n_docs, int64_t *n_words)
{
    (void)n_bytes;
    int64_t cap = 1 << 16;
    WordSlot *tab = (WordSlot *)calloc((size_t)cap, sizeof(WordSlot));
    int64_t maxlen = 1;
    for (int64_t d = 0; d < n_docs; d++)
        if (doc_off[d + 1] - doc_off[d] > maxlen) maxlen = doc_off[d + 1] - doc_off[d];
    int64_t *starts = (int64_t *)malloc(sizeof(int64_t) * (size_t)(maxlen + 1));
    int64_t distinct = 0;
    for (int64_t d = 0; d < n_docs; d++) {
        const uint8_t *doc = data + doc_off[d];
        int64_t n = doc_off[d + 1] - doc_off[d];
        int64_t P = ora_split(doc, n, starts);
        starts[P] = n;
        for (int64_t k = 0; k < P; k++) {
            if (2 * (distinct + 1) > cap) {
                int64_t ncap = 2 * cap, nd = 0;
                WordSlot *nt = (WordSlot *)calloc((size_t)ncap, sizeof(WordSlot));
                for (int64_t i = 0; i < cap; i++)
                    if (tab[i].used) word_insert(nt, ncap, tab[i].p, tab[i].n, tab[i].count, &nd);
                free(tab);
                tab = nt;
                cap = ncap;
            }
            word_insert(tab, cap, doc + starts[k], starts[k + 1] - starts[k], 1, &distinct);
        }
    }
    free(starts);
    Word *words = (Word *)malloc(sizeof(Word) * (size_t)(distinct ? distinct : 1));
    int64_t k = 0;
    for (int64_t i = 0; i < cap; i++) {
        if (!tab[i].used) continue;
        words[k].n = tab[i].n;
        words[k].freq = tab[i].count;
        words[k].sym = (int32_t *)malloc(sizeof(int32_t) * (size_t)(tab[i].n ? tab[i].n : 1));
        for (int64_t j = 0; j < tab[i].n; j++) words[k].sym[j] = tab[i].p[j];
        k++;
    }
    free(tab);
    *n_words = distinct;
    return words;
}

/* Replace every occurrence of (L, Rt) in w by z, left to right without
 * overlap (R4's replacement step).  Returns 1 if anything changed. */
static int replace_pair(Word *w, int32_t L, int32_t Rt, int32_t z)
{
    int64_t o = 0, i = 0;
    int changed = 0;
    while (i < w->n) {
        if (i + 1 < w->n && w->sym[i] == L && w->sym[i + 1] == Rt) {
            w->sym[o++] = z;
            i += 2;
            changed = 1;
        } else {
            w->sym[o++] = w->sym[i++];
        }
    }
    w->n = o;
    return changed;
}

typedef struct {
    uint64_t key;
    int64_t count;
} PairCount;

static int cmp_paircount_key(const void *a, const void *b)
{
    uint64_t x = ((const PairCount *)a)->key, y = ((const PairCount *)b)->key;
    return x < y ? -1 : x > y;
}

/* Naive trainer: a full recount of every pair before every merge, exactly as
 * the step-by-step description reads.  Returns the number of merges made and
 * writes them (and their counts) in rank order. */
static int64_t train_naive(Word *words, int64_t nw, int64_t n_merges,
                           int32_t *merges_out, int64_t *counts_out)
{
    int64_t total = 0;
    for (int64_t i = 0; i < nw; i++) total += words[i].n;
    PairCount *pc = (PairCount *)malloc(sizeof(PairCount) * (size_t)(total ? total : 1));
    int64_t r = 0;
    for (; r < n_merges; r++) {
        int64_t m = 0;
        for (int64_t i = 0; i < nw; i++)
            for (int64_t j = 0; j + 1 < words[i].n; j++) {
                pc[m].key = pkey(words[i].sym[j], words[i].sym[j + 1]);
                pc[m].count = words[i].freq;
                m++;
            }
        if (m == 0) break;
        qsort(pc, (size_t)m, sizeof(PairCount), cmp_paircount_key);
        uint64_t best_key = 0;
        int64_t best = -1;
        for (int64_t a = 0; a < m;) {
            int64_t b = a, c = 0;
            while (b < m && pc[b].key == pc[a].key) c += pc[b++].count;
            /* keys ascend, so a strict '>' keeps the smallest key on ties */
            if (c > best) { best = c; best_key = pc[a].key; }
            a = b;
        }
        if (best < 2) break;
        int32_t L = (int32_t)(best_key >> 32), Rt = (int32_t)(best_key & 0xffffffffu);
        merges_out[2 * r] = L;
        merges_out[2 * r + 1] = Rt;
        if (counts_out) counts_out[r] = best;
        for (int64_t i = 0; i < nw; i++) replace_pair(&words[i], L, Rt, 256 + (int32_t)r);
    }
    free(pc);
    return r;
}

/* --- incremental trainer: same choice rule, counts kept up to date --- */

typedef struct {
    uint64_t key;
    int64_t count;
    int32_t *occ;      /* word indices that may contain the pair */
    int64_t n_occ, cap_occ;
    int64_t stamp;
    int used;
} PairRec;

typedef struct {
    PairRec *slot;
    int64_t cap, n;
} PairMap;

static PairRec *pm_get(PairMap *m, uint64_t key)
{
    if (2 * (m->n + 1) > m->cap) {
        int64_t ncap = m->cap ? 2 * m->cap : 1024;
        PairRec *ns = (PairRec *)calloc((size_t)ncap, sizeof(PairRec));
        for (int64_t i = 0; i < m->cap; i++) {
            if (!m->slot[i].used) continue;
            int64_t j = (int64_t)((m->slot[i].key * 0x9E3779B97F4A7C15ull) >> 20) & (ncap - 1);
            while (ns[j].used) j = (j + 1) & (ncap - 1);
            ns[j] = m->slot[i];
        }
        free(m->slot);
        m->slot = ns;
        m->cap = ncap;
    }
    int64_t j = (int64_t)((key * 0x9E3779B97F4A7C15ull) >> 20) & (m->cap - 1);
    while (m->slot[j].used && m->slot[j].key != key) j = (j + 1) & (m->cap - 1);
    if (!m->slot[j].used) {
        m->slot[j].used = 1;
        m->slot[j].key = key;
        m->slot[j].stamp = -1;
        m->n++;
    }
    return &m->slot[j];
}

static void occ_push(PairRec *p, int32_t w)
{
    if (p->n_occ == p->cap_occ) {
        p->cap_occ = p->cap_occ ? 2 * p->cap_occ : 4;
        p->occ = (int32_t *)realloc(p->occ, sizeof(int32_t) * (size_t)p->cap_occ);
    }
    p->occ[p->n_occ++] = w;
}

typedef struct {
    int64_t count;
    uint64_t key;
} HeapItem;

/* max-heap on (count, then smaller key) */
static int heap_before(const HeapItem *a, const HeapItem *b)
{
    if (a->count != b->count) return a->count > b->count;
    return a->key < b->key;
}

typedef struct {
    HeapItem *v;
    int64_t n, cap;
} Heap;

static void heap_push(Heap *h, int64_t count, uint64_t key)
{
    if (h->n == h->cap) {
        h->cap = h->cap ? 2 * h->cap : 1024;
        h->v = (HeapItem *)realloc(h->v, sizeof(HeapItem) * (size_t)h->cap);
    }
    int64_t i = h->n++;
    h->v[i].count = count;
    h->v[i].key = key;
    while (i > 0) {
        int64_t p = (i - 1) / 2;
        if (!heap_before(&h->v[i], &h->v[p])) break;
        HeapItem t = h->v[i]; h->v[i] = h->v[p]; h->v[p] = t;
        i = p;
    }
}

static HeapItem heap_pop(Heap *h)
{
    HeapItem top = h->v[0];
    h->v[0] = h->v[--h->n];
    int64_t i = 0;
    for (;;) {
        int64_t a = 2 * i + 1, b = a + 1, m = i;
        if (a < h->n && heap_before(&h->v[a], &h->v[m])) m = a;
        if (b < h->n && heap_before(&h->v[b], &h->v[m])) m = b;
        if (m == i) break;
        HeapItem t = h->v[i]; h->v[i] = h->v[m]; h->v[m] = t;
        i = m;
    }
    return top;
}

static int word_has_pair(const Word *w, int32_t L, int32_t Rt)
{
    for (int64_t j = 0; j + 1 < w->n; j++)
        if (w->sym[j] == L && w->sym[j + 1] == Rt) return 1;
    return 0;
}

static int64_t train_incremental(Word *words, int64_t nw, int64_t n_merges,
                                 int32_t *merges_out, int64_t *counts_out)
{
    PairMap pm = {0};
    Heap heap = {0};
    for (int64_t i = 0; i < nw; i++)
        for (int64_t j = 0; j + 1 < words[i].n; j++) {
            PairRec *p = pm_get(&pm, pkey(words[i].sym[j], words[i].sym[j + 1]));
            p->count += words[i].freq;
            if (p->n_occ == 0 || p->occ[p->n_occ - 1] != (int32_t)i) occ_push(p, (int32_t)i);
        }
    for (int64_t s = 0; s < pm.cap; s++)
        if (pm.slot[s].used) heap_push(&heap, pm.slot[s].count, pm.slot[s].key);

    int64_t *wstamp = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nw ? nw : 1));
    for (int64_t i = 0; i < nw; i++) wstamp[i] = -1;
    uint64_t *touched = NULL;
    int64_t n_touched = 0, cap_touched = 0;
    int64_t r = 0;
    for (; r < n_merges; r++) {
        /* current best: pop stale entries until the top matches its pair */
        int64_t best = -1;
        uint64_t best_key = 0;
        while (heap.n > 0) {
            HeapItem it = heap.v[0];
            PairRec *p = pm_get(&pm, it.key);
            if (p->count != it.count) { heap_pop(&heap); continue; }
            best = it.count;
            best_key = it.key;
            break;
        }
        if (best < 2) break;
        int32_t L = (int32_t)(best_key >> 32), Rt = (int32_t)(best_key & 0xffffffffu);
        int32_t z = 256 + (int32_t)r;
        merges_out[2 * r] = L;
        merges_out[2 * r + 1] = Rt;
        if (counts_out) counts_out[r] = best;

        /* copy the occurrence list: pm_get below may move the record */
        PairRec *bp = pm_get(&pm, best_key);
        int64_t n_occ = bp->n_occ;
        int32_t *occ = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n_occ ? n_occ : 1));
        memcpy(occ, bp->occ, sizeof(int32_t) * (size_t)n_occ);
        n_touched = 0;
        for (int64_t a = 0; a < n_occ; a++) {
            int32_t wi = occ[a];
            if (wstamp[wi] == r) continue;
            wstamp[wi] = r;
            Word *w = &words[wi];
            if (!word_has_pair(w, L, Rt)) continue;
            /* remove the word's old pairs, replace, add the new pairs */
            for (int64_t j = 0; j + 1 < w->n; j++) {
                PairRec *p = pm_get(&pm, pkey(w->sym[j], w->sym[j + 1]));
                p->count -= w->freq;
                if (p->stamp != r) {
                    p->stamp = r;
                    if (n_touched == cap_touched) {
                        cap_touched = cap_touched ? 2 * cap_touched : 1024;
                        touched = (uint64_t *)realloc(touched, sizeof(uint64_t) * (size_t)cap_touched);
                    }
                    touched[n_touched++] = p->key;
                }
            }
            replace_pair(w, L, Rt, z);
            for (int64_t j = 0; j + 1 < w->n; j++) {
                PairRec *p = pm_get(&pm, pkey(w->sym[j], w->sym[j + 1]));
                p->count += w->freq;
                if (p->n_occ == 0 || p->occ[p->n_occ - 1] != wi) occ_push(p, wi);
                if (p->stamp != r) {
                    p->stamp = r;
                    if (n_touched == cap_touched) {
                        cap_touched = cap_touched ? 2 * cap_touched : 1024;
                        touched = (uint64_t *)realloc(touched, sizeof(uint64_t) * (size_t)cap_touched);
                    }
                    touched[n_touched++] = p->key;
                }
            }
        }
        free(occ);
        for (int64_t a = 0; a < n_touched; a++) {
            PairRec *p = pm_get(&pm, touched[a]);
            heap_push(&heap, p->count, p->key);
        }
    }
    free(touched);
    free(wstamp);
    for (int64_t s = 0; s < pm.cap; s++) free(pm.slot[s].occ);
    free(pm.slot);
    free(heap.v);
    return r;
}

/* Train up to n_merges merges on a corpus given as documents.  naive != 0
 * selects the full-recount trainer.  Returns the number of merges made. */
int64_t ora_train(const uint8_t *data, int64_t n_bytes, const int64_t *doc_off, int64_t n_docs,
                  int64_t n_merges, int32_t *merges_out, int64_t *counts_out, int naive)
{
    int64_t nw = 0;
    Word *words = collect_words(data, n_bytes, doc_off, n_docs, &nw);
    int64_t r = naive ? train_naive(words, nw, n_merges, merges_out, counts_out)
                      : train_incremental(words, nw, n_merges, merges_out, counts_out);
    for (int64_t i = 0; i < nw; i++) free(words[i].sym);
    free(words);
    return r;
}

/* The trainer's final segmentation of one pre-token is what the encoder must
 * reproduce for it; this entry returns that segmentation by replaying the
 * recorded merges in rank order on the pre-token's bytes (the trainer applies
 * each merge to every word as it is chosen).  Returns the symbol count. */
int64_t ora_replay_merges(const int32_t *merges, int64_t R, const uint8_t *w, int64_t n, int32_t *out)
{
    Word x;
    x.sym = out;
    x.n = n;
    x.freq = 1;
    for (int64_t i = 0; i < n; i++) out[i] = w[i];
    for (int64_t r = 0; r < R; r++) replace_pair(&x, merges[2 * r], merges[2 * r + 1], 256 + (int32_t)r);
    return x.n;
}
