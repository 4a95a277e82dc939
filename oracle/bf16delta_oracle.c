/*
 * bf16delta_oracle.c -- TEST INFRASTRUCTURE ONLY (see bf16delta_oracle.h).
 *
 * Plain single-threaded C, one element at a time, in the order the format
 * defines things.  No blocking, no fusion, no reordering beyond what the
 * definition states, so that it can be read against the pages by eye:
 *
 *   encode (compress), per block of 8192 elements:
 *     1. x = old XOR new for every element           (Weight Teleportation,
 *        "Delta update algebra")
 *     2. class U (x == 0), M (only bits 0..6 set), R (any of bits 7..15 set)
 *                                                     (ARCv3 blog, "Deep dive
 *        into ARCv3": mantissa-only vs exponent/sign changes)
 *     3. U is dropped; the changed positions go into a position segment
 *        (gap list or bitmap, whichever is smaller); every changed element
 *        contributes a 7-bit mantissa field (its mantissa XOR, or 0 if it is
 *        R); every R element contributes its whole 16-bit XOR word to the
 *        rare segment                                 (ARCv3 blog, figure "How
 *        ARCv3 encodes a block of weights")
 *   checksum of the new weights, returned beside the payload (ARCv3 blog,
 *   "Deep dive into ARCv3" and "Using ARCv3").
 *
 *   decode (decompress): validate, XOR the decoded mask onto the old weights
 *   in place, verify the checksum; on any failure XOR the same mask again
 *   (XOR is its own inverse, "Delta update algebra") so the weights end as
 *   the old ones bit for bit.
 *
 *   version 2 (Weight Teleportation, "Eval, fault tolerance, and resuming
 *   from trained checkpoints": deltas between versions other than the last
 *   one; the Delta-Compressed Refit summary: absolute overwrites beside XOR
 *   masks, retry-safe versioning with a joint commit): the header also binds
 *   the payload to a base and a target version, and an overwrite payload
 *   carries each changed element's new value instead of its XOR.  The
 *   receiver's version word must equal the base before anything is touched,
 *   and becomes the target only together with the new weights.
 */
#include "bf16delta_oracle.h"

#include <stdlib.h>
#include <string.h>

/* ---- format constants (bf16delta_v1) ---------------------------------- */
#define BLOCK_ELEMS     8192u
#define HEADER_BYTES    64u
#define FORMAT_VERSION  1u
/* version 2: a 32-byte binding block follows the v1 header fields */
#define FORMAT_VERSION_BOUND 2u
#define HEADER_BYTES_V2 96u
#define FLAG_OVERWRITE  1u
#define CODE_BITMAP     15u
#define CODE_INVALID    14u
#define EXP_SIGN_BITS   0xFF80u   /* sign (bit 15) and exponent (bits 7..14) */
#define MANT_BITS       0x007Fu   /* mantissa (bits 0..6) */
static const char MAGIC[8] = {'B', 'F', '1', '6', 'D', 'X', 'O', 'R'};

/* ---- small helpers ---------------------------------------------------- */
static uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

/* number of bits needed to write v (0 for v == 0) */
static unsigned bit_length(uint64_t v) {
    unsigned len = 0;
    while (v) { len++; v >>= 1; }
    return len;
}

static void put_u32(uint8_t *p, uint32_t v) {
    for (int i = 0; i < 4; i++) p[i] = (uint8_t)(v >> (8 * i));
}
static void put_u64(uint8_t *p, uint64_t v) {
    for (int i = 0; i < 8; i++) p[i] = (uint8_t)(v >> (8 * i));
}
static uint32_t get_u32(const uint8_t *p) {
    uint32_t v = 0;
    for (int i = 0; i < 4; i++) v |= (uint32_t)p[i] << (8 * i);
    return v;
}
static uint64_t get_u64(const uint8_t *p) {
    uint64_t v = 0;
    for (int i = 0; i < 8; i++) v |= (uint64_t)p[i] << (8 * i);
    return v;
}

/* LSB-first bit writer: bit t of a field written at stream bit o lands in
 * stream bit o + t; stream bit k is bit (k mod 8) of byte k / 8.  The
 * buffer must be zeroed beforehand, so padding bits stay zero. */
static void put_bits(uint8_t *buf, uint64_t bitpos, uint32_t value, unsigned width) {
    for (unsigned t = 0; t < width; t++) {
        if ((value >> t) & 1u) {
            uint64_t k = bitpos + t;
            buf[k / 8] |= (uint8_t)(1u << (k % 8));
        }
    }
}
static uint32_t get_bits(const uint8_t *buf, uint64_t bitpos, unsigned width) {
    uint32_t v = 0;
    for (unsigned t = 0; t < width; t++) {
        uint64_t k = bitpos + t;
        if ((buf[k / 8] >> (k % 8)) & 1u) v |= 1u << t;
    }
    return v;
}

/* ---- element classification (ARCv3 blog, "Deep dive into ARCv3") ------ */
enum { CLASS_U = 0, CLASS_M = 1, CLASS_R = 2 };
static int classify(uint16_t x) {
    if (x == 0) return CLASS_U;                 /* unchanged: omitted           */
    if ((x & EXP_SIGN_BITS) == 0) return CLASS_M;  /* only mantissa bits flipped */
    return CLASS_R;                             /* exponent or sign flipped     */
}

/* ---- checksum ---------------------------------------------------------
 * The pages ask for a checksum of the trainer's weights that the receiver
 * compares against (ARCv3 blog, "Deep dive into ARCv3"); they name no
 * algorithm.  bf16delta_v1 uses the SplitMix64 finaliser (Steele, Lea and
 * Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014, with
 * Stafford's "Mix13" constants) over 64-bit words:
 *   W_k = little-endian u64 of elements 4k..4k+3 (missing elements are 0)
 *   S   = sum over k of mix64(W_k XOR (k+1)*G)  mod 2^64,  G = 0x9E3779B97F4A7C15
 *   checksum = mix64(S XOR n)                                              */
#define GOLDEN_GAMMA 0x9E3779B97F4A7C15ull

uint64_t bf16d_ref_mix64(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ull;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBull;
    z ^= z >> 31;
    return z;
}

uint64_t bf16d_ref_checksum(const uint16_t *w, uint64_t n) {
    uint64_t sum = 0;
    uint64_t n_words = ceil_div(n, 4);
    for (uint64_t k = 0; k < n_words; k++) {
        uint64_t word = 0;
        for (unsigned t = 0; t < 4; t++) {
            uint64_t i = 4 * k + t;
            uint64_t e = (i < n) ? w[i] : 0;
            word |= e << (16 * t);
        }
        sum += bf16d_ref_mix64(word ^ ((k + 1) * GOLDEN_GAMMA));
    }
    return bf16d_ref_mix64(sum ^ n);
}

/* ---- sizes ------------------------------------------------------------- */
static uint64_t block_len(uint64_t n, uint64_t b) {
    uint64_t start = b * BLOCK_ELEMS;
    uint64_t end = start + BLOCK_ELEMS;
    if (end > n) end = n;
    return end - start;
}

static uint64_t pos_segment_bytes(uint32_t code, uint64_t c, uint64_t L) {
    if (code == CODE_BITMAP) return ceil_div(L, 8);
    return ceil_div(c * code, 8);
}
static uint64_t mant_segment_bytes(uint64_t c) { return ceil_div(7 * c, 8); }
static uint64_t rare_segment_bytes(uint64_t r) { return 2 * r; }

/* An overwrite record has no mantissa segment: its word segment holds the
 * new value of every changed element (r == c). */
static uint64_t mant_bytes_mode(uint64_t c, int overwrite) {
    return overwrite ? 0 : mant_segment_bytes(c);
}

uint64_t bf16d_ref_max_payload_bytes(uint64_t n) {
    /* per block: position segment <= bitmap size (the smaller encoding is
     * always taken), every element changed and rare for the value streams */
    uint64_t nb = ceil_div(n, BLOCK_ELEMS);
    uint64_t total = HEADER_BYTES + 4 * nb;
    for (uint64_t b = 0; b < nb; b++) {
        uint64_t L = block_len(n, b);
        total += ceil_div(L, 8) + mant_segment_bytes(L) + rare_segment_bytes(L);
    }
    return total;
}

/* ---- encoder ----------------------------------------------------------- */

/* One block: fills rec[] (zeroed by the caller, >= 3*8192+2 bytes), returns
 * the record length and the descriptor. */
static uint64_t encode_block(const uint16_t *src, const uint16_t *dst, uint64_t L,
                             int overwrite, uint8_t *rec, uint32_t *desc_out,
                             uint64_t *c_out, uint64_t *r_out, int *is_bitmap) {
    uint16_t pos[BLOCK_ELEMS];
    uint16_t val[BLOCK_ELEMS];
    uint64_t c = 0, r = 0;

    /* steps 1-2: XOR and classify, keeping changed elements in order */
    for (uint64_t j = 0; j < L; j++) {
        uint16_t x = (uint16_t)(src[j] ^ dst[j]);
        int cls = classify(x);
        if (cls == CLASS_U) continue;
        pos[c] = (uint16_t)j;
        val[c] = x;
        c++;
        if (cls == CLASS_R) r++;
    }

    /* step 3: gaps, their width, and the cheaper position encoding */
    uint64_t max_gap = 0;
    for (uint64_t j = 0; j < c; j++) {
        uint64_t gap = (j == 0) ? pos[0] : (uint64_t)(pos[j] - pos[j - 1] - 1);
        if (gap > max_gap) max_gap = gap;
    }
    unsigned w = bit_length(max_gap);
    uint64_t delta_bytes = ceil_div(c * w, 8);
    uint64_t bitmap_bytes = ceil_div(L, 8);
    uint32_t code = (bitmap_bytes < delta_bytes) ? CODE_BITMAP : w;

    /* position segment */
    uint64_t pb = pos_segment_bytes(code, c, L);
    if (code == CODE_BITMAP) {
        for (uint64_t j = 0; j < c; j++) put_bits(rec, pos[j], 1, 1);
    } else {
        for (uint64_t j = 0; j < c; j++) {
            uint64_t gap = (j == 0) ? pos[0] : (uint64_t)(pos[j] - pos[j - 1] - 1);
            put_bits(rec, j * w, (uint32_t)gap, w);
        }
    }

    if (overwrite) {
        /* word segment: the absolute new value of every changed element */
        uint8_t *words = rec + pb;
        for (uint64_t j = 0; j < c; j++) {
            uint16_t v = dst[pos[j]];
            words[2 * j] = (uint8_t)(v & 0xFF);
            words[2 * j + 1] = (uint8_t)(v >> 8);
        }
        *desc_out = (uint32_t)c | ((uint32_t)c << 14) | (code << 28);
        *c_out = c;
        *r_out = c;
        *is_bitmap = (code == CODE_BITMAP);
        return pb + rare_segment_bytes(c);
    }

    /* mantissa segment: 7-bit mantissa XOR, 0 = "see the rare stream" */
    uint64_t mb = mant_segment_bytes(c);
    for (uint64_t j = 0; j < c; j++) {
        uint32_t field = (classify(val[j]) == CLASS_M) ? (val[j] & MANT_BITS) : 0;
        put_bits(rec + pb, 7 * j, field, 7);
    }

    /* rare segment: the whole XOR word of every exponent/sign change */
    uint8_t *rare = rec + pb + mb;
    uint64_t k = 0;
    for (uint64_t j = 0; j < c; j++) {
        if (classify(val[j]) != CLASS_R) continue;
        rare[2 * k] = (uint8_t)(val[j] & 0xFF);
        rare[2 * k + 1] = (uint8_t)(val[j] >> 8);
        k++;
    }

    *desc_out = (uint32_t)c | ((uint32_t)r << 14) | (code << 28);
    *c_out = c;
    *r_out = r;
    *is_bitmap = (code == CODE_BITMAP);
    return pb + mb + rare_segment_bytes(r);
}

/* bound: 0 writes a version-1 payload; otherwise version 2 with the given
 * binding and flags. */
static int compress_any(const uint16_t *src, const uint16_t *dst, uint64_t n, int bound,
                        uint64_t base_version, uint64_t target_version, uint32_t flags,
                        uint8_t *payload, uint64_t capacity, ref_result *res) {
    if (res == NULL) return REF_EINVAL;
    memset(res, 0, sizeof(*res));
    if (n > 0 && (src == NULL || dst == NULL)) return REF_EINVAL;
    if (payload == NULL && capacity > 0) return REF_EINVAL;
    if ((flags & ~FLAG_OVERWRITE) != 0 || (!bound && flags != 0)) return REF_EINVAL;
    const int overwrite = (flags & FLAG_OVERWRITE) != 0;
    const uint64_t hdr = bound ? HEADER_BYTES_V2 : HEADER_BYTES;

    uint64_t nb = ceil_div(n, BLOCK_ELEMS);
    uint64_t data_off = hdr + 4 * nb;
    uint8_t *rec = (uint8_t *)malloc(3 * BLOCK_ELEMS + 16);
    if (rec == NULL) return REF_EINVAL;

    uint64_t off = data_off;
    uint64_t n_changed = 0, n_rare = 0, n_bitmap = 0;
    uint64_t pos_total = 0, mant_total = 0, rare_total = 0;
    for (uint64_t b = 0; b < nb; b++) {
        uint64_t L = block_len(n, b);
        uint32_t desc;
        uint64_t c, r;
        int is_bitmap;
        memset(rec, 0, 3 * BLOCK_ELEMS + 16);
        uint64_t len = encode_block(src + b * BLOCK_ELEMS, dst + b * BLOCK_ELEMS, L,
                                    overwrite, rec, &desc, &c, &r, &is_bitmap);
        /* descriptor table entry b, then the record at the running offset;
         * nothing is written at or beyond capacity */
        uint64_t desc_at = hdr + 4 * b;
        if (desc_at + 4 <= capacity) put_u32(payload + desc_at, desc);
        for (uint64_t i = 0; i < len; i++)
            if (off + i < capacity) payload[off + i] = rec[i];
        off += len;

        n_changed += c;
        n_rare += r;
        n_bitmap += (uint64_t)is_bitmap;
        pos_total += pos_segment_bytes(desc >> 28, c, L);
        mant_total += mant_bytes_mode(c, overwrite);
        rare_total += rare_segment_bytes(r);
    }
    free(rec);

    res->payload_bytes = off;
    res->checksum = bf16d_ref_checksum(dst, n);
    res->n_changed = n_changed;
    res->n_rare = n_rare;
    res->n_bitmap_blocks = n_bitmap;
    if (off > capacity) return REF_ECAPACITY;

    /* header */
    memcpy(payload, MAGIC, 8);
    put_u32(payload + 8, bound ? FORMAT_VERSION_BOUND : FORMAT_VERSION);
    put_u32(payload + 12, BLOCK_ELEMS);
    put_u64(payload + 16, n);
    put_u64(payload + 24, n_changed);
    put_u64(payload + 32, n_rare);
    put_u64(payload + 40, pos_total);
    put_u64(payload + 48, mant_total);
    put_u64(payload + 56, rare_total);
    if (bound) {
        put_u64(payload + 64, base_version);
        put_u64(payload + 72, target_version);
        put_u32(payload + 80, flags);
        put_u32(payload + 84, 0);
        put_u64(payload + 88, 0);
    }
    return REF_OK;
}

int bf16d_ref_compress(const uint16_t *src, const uint16_t *dst, uint64_t n,
                       uint8_t *payload, uint64_t capacity, ref_result *res) {
    return compress_any(src, dst, n, 0, 0, 0, 0, payload, capacity, res);
}

int bf16d_ref_compress_v2(const uint16_t *src, const uint16_t *dst, uint64_t n,
                          uint64_t base_version, uint64_t target_version, uint32_t flags,
                          uint8_t *payload, uint64_t capacity, ref_result *res) {
    return compress_any(src, dst, n, 1, base_version, target_version, flags, payload,
                        capacity, res);
}

/* ---- decoder ----------------------------------------------------------- */

/* Decode and check one block record; on success fill pos[]/val[] (c entries)
 * and return 1, on any malformation return 0. */
static int decode_block(const uint8_t *rec, uint32_t desc, uint64_t L, int overwrite,
                        uint16_t *pos, uint16_t *val) {
    uint64_t c = desc & 0x3FFFu;
    uint64_t r = (desc >> 14) & 0x3FFFu;
    uint32_t code = desc >> 28;
    uint64_t pb = pos_segment_bytes(code, c, L);
    uint64_t mb = mant_bytes_mode(c, overwrite);
    const uint8_t *mant = rec + pb;
    const uint8_t *rare = rec + pb + mb;

    /* positions */
    if (code == CODE_BITMAP) {
        uint64_t found = 0;
        for (uint64_t j = 0; j < L; j++) {
            if (get_bits(rec, j, 1)) {
                if (found < c) pos[found] = (uint16_t)j;
                found++;
            }
        }
        if (found != c) return 0;
        for (uint64_t k = L; k < 8 * pb; k++)
            if (get_bits(rec, k, 1)) return 0;            /* pad bits must be 0 */
        /* canonical: the bitmap must be strictly smaller than the gap list */
        uint64_t max_gap = 0;
        for (uint64_t j = 0; j < c; j++) {
            uint64_t gap = (j == 0) ? pos[0] : (uint64_t)(pos[j] - pos[j - 1] - 1);
            if (gap > max_gap) max_gap = gap;
        }
        if (!(ceil_div(L, 8) < ceil_div(c * bit_length(max_gap), 8))) return 0;
    } else {
        unsigned w = code;
        uint64_t p = 0, max_gap = 0;
        for (uint64_t j = 0; j < c; j++) {
            uint64_t gap = get_bits(rec, j * w, w);
            p = (j == 0) ? gap : p + gap + 1;
            if (p >= L) return 0;                          /* position out of block */
            pos[j] = (uint16_t)p;
            if (gap > max_gap) max_gap = gap;
        }
        if (bit_length(max_gap) != w) return 0;           /* width must be minimal */
        for (uint64_t k = c * w; k < 8 * pb; k++)
            if (get_bits(rec, k, 1)) return 0;
    }

    /* overwrite record: the absolute new values, one word per position */
    if (overwrite) {
        for (uint64_t j = 0; j < c; j++)
            val[j] = (uint16_t)(mant[2 * j] | (mant[2 * j + 1] << 8));
        return 1;
    }

    /* values: mantissa fields, zero escapes into the rare words */
    uint64_t next_rare = 0;
    for (uint64_t j = 0; j < c; j++) {
        uint32_t field = get_bits(mant, 7 * j, 7);
        if (field != 0) {
            val[j] = (uint16_t)field;
        } else {
            if (next_rare >= r) return 0;
            uint16_t x = (uint16_t)(rare[2 * next_rare] | (rare[2 * next_rare + 1] << 8));
            if ((x & EXP_SIGN_BITS) == 0) return 0;        /* must really be rare */
            val[j] = x;
            next_rare++;
        }
    }
    if (next_rare != r) return 0;
    for (uint64_t k = 7 * c; k < 8 * mb; k++)
        if (get_bits(mant, k, 1)) return 0;
    return 1;
}

/* XOR every well-formed block's mask onto the weights; returns the number of
 * malformed blocks (which are left alone).  Running it twice is a no-op. */
static uint64_t apply_pass(uint16_t *weights, uint64_t n, const uint8_t *payload,
                           uint64_t hdr, int overwrite) {
    uint16_t pos[BLOCK_ELEMS];
    uint16_t val[BLOCK_ELEMS];
    uint64_t nb = ceil_div(n, BLOCK_ELEMS);
    uint64_t off = hdr + 4 * nb;
    uint64_t bad = 0;
    for (uint64_t b = 0; b < nb; b++) {
        uint64_t L = block_len(n, b);
        uint32_t desc = get_u32(payload + hdr + 4 * b);
        uint64_t c = desc & 0x3FFFu, r = (desc >> 14) & 0x3FFFu;
        uint64_t len = pos_segment_bytes(desc >> 28, c, L) + mant_bytes_mode(c, overwrite) +
                       rare_segment_bytes(r);
        if (decode_block(payload + off, desc, L, overwrite, pos, val)) {
            for (uint64_t j = 0; j < c; j++) {
                if (overwrite)
                    weights[b * BLOCK_ELEMS + pos[j]] = val[j];   /* absolute value */
                else
                    weights[b * BLOCK_ELEMS + pos[j]] ^= val[j];  /* XOR mask */
            }
        } else {
            bad++;
        }
        off += len;
    }
    return bad;
}

int bf16d_ref_decompress_v2(uint16_t *weights, uint64_t n, const uint8_t *payload,
                            uint64_t payload_bytes, uint64_t checksum, uint64_t *version) {
    if ((payload == NULL && payload_bytes > 0) || (n > 0 && weights == NULL)) return REF_EINVAL;

    /* header: version 1, or version 2 with its binding block */
    if (payload_bytes < HEADER_BYTES) return REF_EFORMAT;
    if (memcmp(payload, MAGIC, 8) != 0) return REF_EFORMAT;
    uint32_t fv = get_u32(payload + 8);
    if (fv != FORMAT_VERSION && fv != FORMAT_VERSION_BOUND) return REF_EFORMAT;
    const int bound = fv == FORMAT_VERSION_BOUND;
    const uint64_t hdr = bound ? HEADER_BYTES_V2 : HEADER_BYTES;
    if (payload_bytes < hdr) return REF_EFORMAT;
    if (get_u32(payload + 12) != BLOCK_ELEMS) return REF_EFORMAT;
    if (get_u64(payload + 16) != n) return REF_EFORMAT;
    uint64_t base_version = 0, target_version = 0;
    uint32_t flags = 0;
    if (bound) {
        base_version = get_u64(payload + 64);
        target_version = get_u64(payload + 72);
        flags = get_u32(payload + 80);
        if ((flags & ~FLAG_OVERWRITE) != 0) return REF_EFORMAT;
        if (get_u32(payload + 84) != 0 || get_u64(payload + 88) != 0) return REF_EFORMAT;
    }
    const int overwrite = (flags & FLAG_OVERWRITE) != 0;
    uint64_t nb = ceil_div(n, BLOCK_ELEMS);
    if (payload_bytes < hdr + 4 * nb) return REF_EFORMAT;

    /* descriptor table: each entry well formed and in canonical mode, and
     * the totals agree with the header and with the payload length */
    uint64_t sum_c = 0, sum_r = 0, sum_pos = 0, sum_mant = 0, sum_rare = 0;
    for (uint64_t b = 0; b < nb; b++) {
        uint64_t L = block_len(n, b);
        uint32_t desc = get_u32(payload + hdr + 4 * b);
        uint64_t c = desc & 0x3FFFu, r = (desc >> 14) & 0x3FFFu;
        uint32_t code = desc >> 28;
        if (code == CODE_INVALID) return REF_EFORMAT;
        if (c > L || r > c) return REF_EFORMAT;
        if (overwrite && r != c) return REF_EFORMAT;   /* one word per change */
        if (code == CODE_BITMAP) {
            if (c == 0) return REF_EFORMAT;
        } else {
            if (c == 0 && code != 0) return REF_EFORMAT;
            if (ceil_div(c * code, 8) > ceil_div(L, 8)) return REF_EFORMAT;
        }
        sum_c += c;
        sum_r += r;
        sum_pos += pos_segment_bytes(code, c, L);
        sum_mant += mant_bytes_mode(c, overwrite);
        sum_rare += rare_segment_bytes(r);
    }
    if (sum_c != get_u64(payload + 24) || sum_r != get_u64(payload + 32) ||
        sum_pos != get_u64(payload + 40) || sum_mant != get_u64(payload + 48) ||
        sum_rare != get_u64(payload + 56))
        return REF_EFORMAT;
    if (hdr + 4 * nb + sum_pos + sum_mant + sum_rare != payload_bytes)
        return REF_EFORMAT;

    /* the binding: a version-2 payload applies only to the version it was
     * made against; nothing is touched otherwise */
    if (bound && version != NULL && *version != base_version) return REF_EVERSION;

    if (overwrite) {
        /* absolute values cannot be undone by applying them again, so the
         * result is built and checked in a copy, and written back only when
         * it is right */
        uint16_t *tmp = (uint16_t *)malloc(2 * n + 2);
        if (tmp == NULL) return REF_EINVAL;
        if (n) memcpy(tmp, weights, 2 * n);
        uint64_t bad = apply_pass(tmp, n, payload, hdr, 1);
        int st = REF_OK;
        if (bad != 0) st = REF_EFORMAT;
        else if (bf16d_ref_checksum(tmp, n) != checksum) st = REF_ECHECKSUM;
        if (st == REF_OK && n) memcpy(weights, tmp, 2 * n);
        free(tmp);
        if (st != REF_OK) return st;
    } else {
        /* apply; a malformed block or a checksum mismatch undoes the pass */
        uint64_t bad = apply_pass(weights, n, payload, hdr, 0);
        if (bad != 0) {
            apply_pass(weights, n, payload, hdr, 0);
            return REF_EFORMAT;
        }
        if (bf16d_ref_checksum(weights, n) != checksum) {
            apply_pass(weights, n, payload, hdr, 0);
            return REF_ECHECKSUM;
        }
    }
    /* joint commit: the weights and the version word move together */
    if (bound && version != NULL) *version = target_version;
    return REF_OK;
}

int bf16d_ref_decompress(uint16_t *weights, uint64_t n, const uint8_t *payload,
                         uint64_t payload_bytes, uint64_t checksum) {
    return bf16d_ref_decompress_v2(weights, n, payload, payload_bytes, checksum, NULL);
}
