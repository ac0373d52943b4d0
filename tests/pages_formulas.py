"""Closed forms the PipeSpec review states, written out for the tests.

* Expected tokens emitted by one verification window of gamma drafts with a
  constant per-token acceptance alpha: (1 - alpha^(gamma+1)) / (1 - alpha),
  the Leviathan et al. formula the review uses ("Assumptions & free
  parameters", second item; "Core claim").
* Recurrence of the probability that stage i verifies at step j and its
  steady state rho = alpha / (1 - alpha^(gamma+1) + alpha) ("What carries the
  argument").
* E[N] = (1 - rho) * 1 + rho * (1 - alpha^(gamma+1)) / (1 - alpha) > 1
  ("What carries the argument"; Theorem 1 in "Core claim").
"""


def expected_tokens_per_window(alpha, gamma):
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def rho_step(rho_prev, alpha, gamma):
    return rho_prev * alpha ** (gamma + 1) + (1.0 - rho_prev) * alpha


def rho_steady(alpha, gamma):
    return alpha / (1.0 - alpha ** (gamma + 1) + alpha)


def expected_tokens_per_step(alpha, gamma):
    rho = rho_steady(alpha, gamma)
    return (1.0 - rho) * 1.0 + rho * expected_tokens_per_window(alpha, gamma)


def truncated_geometric(alpha, gamma):
    """Law of the number n of accepted drafts in a gamma-window when each draft
    is accepted independently with probability alpha and the scan stops at the
    first rejection."""
    return [alpha ** k * (1 - alpha) for k in range(gamma)] + [alpha ** gamma]
